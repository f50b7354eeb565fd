"""Decode batches regrouped by expert affinity (moe_group_tokens) give every
token the same output, bit for bit, as arrival-order batches of the same
size (tokens are independent and the batch size fixes the kernels' plan),
and activate fewer distinct experts on skewed routing."""
import numpy as np
import pytest
import torch

import workloads as wl
from gpu_common import Layer, dev, lib
from oracle import grouping as og

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.mark.parametrize("alpha", [0.0, 1.5])
def test_grouped_batches_match_arrival_batches(alpha):
    spec = wl.TINY.with_(T=256, d=512, f=256, E=128, k=8, bias="zipf", bias_param=alpha)
    L = Layer(spec, want_oracle=False)
    layer = L.layer()
    m = lib()
    ids = torch.empty((spec.T, spec.k), dtype=torch.int32, device=dev())
    layer.forward(L.x, topk_ids=ids)
    ids_np = ids.cpu().numpy()
    B = 64
    order = m.group_tokens(ids_np, spec.E, B)
    assert np.array_equal(order, og.group_tokens(ids_np, B))

    def run(idx):
        out = torch.empty((spec.T, spec.d), dtype=torch.float32, device=dev())
        for b in range(0, spec.T, B):
            sel = torch.as_tensor(idx[b:b + B], device=dev(), dtype=torch.long)
            out[sel] = layer.forward(L.x[sel].contiguous())
        torch.cuda.synchronize()
        return out

    arrival = run(np.arange(spec.T))
    grouped = run(order)
    assert torch.equal(arrival, grouped)
    d_arr = og.distinct_per_batch(ids_np, np.arange(spec.T), B)
    d_grp = og.distinct_per_batch(ids_np, order, B)
    assert sum(d_grp) <= sum(d_arr)
    if alpha > 0:
        assert sum(d_grp) < sum(d_arr)
