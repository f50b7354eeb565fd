"""Decode time follows the distinct experts a batch activates ("ELDR : Microsoft
et KAIST accélèrent le décodage des MoE", first paragraph: every decode step
loads the weights of each distinct expert its batch routes to).  On the
Qwen3-30B-A3B-shaped layer at T=64 the Zipf router offsets calibrated for 16,
64 and 96 distinct experts, and no offset (~127), must give layer times that
grow with the number of experts, by at least half again from 16 to ~127 (the
weight bytes grow ~8x; the fixed launch costs keep the ratio well below that).
A qualitative check: one timing per point after a warm-up, median of 20."""
import pytest
import torch

import workloads as wl
from gpu_common import Layer, dev, lib

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _median_us(layer, x, bias, steps=20, warmup=5):
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    out = torch.empty((x.shape[0], layer.w.d), dtype=torch.float32, device=dev())
    for _ in range(warmup):
        layer.forward(x, out=out)
    for a, b in ev:
        a.record()
        layer.forward(x, out=out)
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)
    return t[len(t) // 2]


def test_decode_time_grows_with_distinct_experts():
    spec = wl.QWEN3.with_(T=64, bias="none")
    L = Layer(spec, want_oracle=False)
    m = lib()
    times, distinct = [], []
    for D in (16, 64, 96, None):
        b = None if D is None else wl.zipf_bias(wl.QWEN3.with_(bias_param=wl.qwen3_alpha(D)), 0)
        b = None if b is None else b.to(dev())
        layer = m.MoELayer(L.dw, L.w_router, spec.k, router_bias=b)
        ids = torch.empty((spec.T, spec.k), dtype=torch.int32, device=dev())
        layer.forward(L.x, topk_ids=ids)
        torch.cuda.synchronize()
        distinct.append(int(torch.unique(ids).numel()))
        times.append(_median_us(layer, L.x, b))
    print("distinct experts", distinct, "median us", [round(t, 1) for t in times])
    assert distinct == sorted(distinct) and distinct[0] <= 16 < distinct[-1]
    assert all(a < b for a, b in zip(times, times[1:])), (distinct, times)
    assert times[-1] >= 1.5 * times[0], (distinct, times)
