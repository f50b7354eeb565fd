"""The fused layer captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capture stream): every replay must equal the eager
forward on the same input, bit for bit, with eager work, input changes and
synchronisations between the replays.  The layer's launches are kernels
only (no memset, allocation or synchronisation), which is what makes them
capturable; the workspace and the output are allocated before capture."""
import pytest
import torch

import workloads as wl
from gpu_common import Layer, dev

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SPECS = {
    "tiny": wl.TINY,
    "zipf-two-shapes": wl.TINY.with_(T=64, d=512, f=256, E=128, k=8, bias="zipf", bias_param=2.0),
    "shared-elastic": wl.TINY.with_(T=48, d=256, f=192, E=16, k=4, n_shared=2, k_choices=(1, 2, 4)),
    # routing by two tokens x four experts per wave, and in one prefill launch
    "mid-routing": wl.TINY.with_(T=301, d=256, f=128, E=70, k=6, k_choices=(2, 4, 6)),
    "prefill-routing": wl.TINY.with_(T=1100, d=256, f=128, E=64, k=6, n_shared=1),
}


def _capture(layer, x, kpt, out):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(x, k_per_token=kpt, out=out)  # workspace allocated before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(x, k_per_token=kpt, out=out)
    return g


@pytest.mark.parametrize("name", list(SPECS))
@pytest.mark.parametrize("msub", [None, 16])
def test_graph_replays_match_eager(name, msub, monkeypatch):
    if msub is not None:
        monkeypatch.setenv("FP8MOE_MSUB", str(msub))  # 256-row passes as at prefill
    L = Layer(SPECS[name], want_oracle=False)
    layer = L.layer()
    x = L.x.clone()
    out = torch.empty((x.shape[0], L.spec.d), dtype=torch.float32, device=dev())
    g = _capture(layer, x, L.kpt, out)
    gen = torch.Generator(device=dev()).manual_seed(7)
    for rep in range(4):
        if rep % 2 == 1:  # a new input in the captured buffer
            x.copy_(torch.randn(x.shape, generator=gen, device=dev()))
        g.replay()
        torch.cuda.synchronize()
        eager = layer.forward(x.clone(), k_per_token=L.kpt)  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager forward"
    del g


# ------------------------------------------------------------------ one graph per k
# The MoE-Prism page (section Méthodologie B, segmented graph executor): the
# MoE segment of a block is captured once per routing budget k and replayed
# for batches served at that k.  Here: one graph per k of the elastic-k layer
# shape, replays interleaved across k with new inputs in the captured
# buffers, every replay compared with the oracle on every token.

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from gpu_common import lib, rel_l2, to_np  # noqa: E402

PER_K = {
    "prism-small": (wl.PRISM.with_(T=96, d=256, E=64, k_choices=()), (4, 8, 16, 32)),
    "prism": (wl.PRISM.with_(k_choices=()), (4, 8, 16, 32)),
}


@pytest.mark.parametrize("name", list(PER_K))
def test_graph_per_k_matches_oracle(name):
    spec, ks = PER_K[name]
    L = Layer(spec)
    gen = torch.Generator(device=dev()).manual_seed(11)
    graphs = {}
    for k in ks:
        layer = lib().MoELayer(L.dw, L.w_router, k)
        x = L.x.clone()
        out = torch.empty((spec.T, spec.d), dtype=torch.float32, device=dev())
        ids = torch.empty((spec.T, k), dtype=torch.int32, device=dev())
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            layer.forward(x, out=out, topk_ids=ids)  # workspace allocated before capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.forward(x, out=out, topk_ids=ids)
        graphs[k] = (g, layer, x, out, ids)
    for rep in range(3):
        for k in ks:
            g, layer, x, out, ids = graphs[k]
            if rep > 0:  # a new batch in the captured input buffer
                x.copy_(torch.randn(x.shape, generator=gen, device=dev()))
            g.replay()
            torch.cuda.synchronize()
            eager = layer.forward(x.clone())  # eager work between replays
            lo = to_np(lib().router_logits(x, L.w_router))
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"k={k} replay {rep}: differs from eager"
            ref, ido, _ = oracle.forward(to_np(x), L.qw, k, logits_override=lo)
            np.testing.assert_array_equal(to_np(ids), ido)
            got = to_np(out)
            err = rel_l2(got, ref)
            per = np.linalg.norm(got - ref, axis=1) / np.linalg.norm(ref, axis=1)
            assert err <= 2e-2 and per.max() <= 2e-2, (k, rep, err, per.max())
            print(f"{name} k={k} replay {rep}: rel-L2 {err:.3e}, worst token {per.max():.3e}")
    del graphs
