"""The gate/up GEMM with the per-row e4m3 requantisation fused into its
SiLU*up epilogue, used where one workgroup's channels span a row's whole f
(f <= 192, e.g. the MoE-Prism sub-experts with f = 192).

The fused epilogue forms h with the same operations as the h epilogue and
requantises it with the separate requantisation's operations, so the layer's
output must be the same bit for bit as with the separate launch
(FP8MOE_RQ=0), at every row-pass height, and every token within the bar
against the oracle ("Routage MoE entre GPU": the layer statement the oracle
implements).
"""
import numpy as np
import pytest
import torch

import workloads as wl
import oracle
from gpu_common import Layer, dev, lib, rel_l2, to_np
from test_gpu_layer import TOL_REQUANT, _check, row_rel_l2

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

RQ_SPECS = {
    # variable k, 64 experts: short items of a few rows
    "f192-elastic": wl.TINY.with_(T=77, d=256, f=192, E=64, k=32, k_choices=(4, 8, 16, 32)),
    # shared experts (rows past the routed capacity), two channel-group waves
    "f64-shared": wl.TINY.with_(T=40, d=512, f=64, E=8, k=2, n_shared=2),
    # ragged d: two and a half K steps (a 64-byte K tail)
    "f192-ragged": wl.TINY.with_(T=19, d=320, f=192, E=5, k=3),
    # long items (about 50 rows of one expert in a 128-row pass)
    "f192-long": wl.TINY.with_(T=100, d=256, f=192, E=4, k=2),
    # four waves
    "f128-long": wl.TINY.with_(T=100, d=256, f=128, E=4, k=2),
}
# Against the oracle: the batch within the bar for every spec, and every
# token on its own for all but the two four-expert "long" layers (d = 256,
# rows of 128 and 192 values).  There one e4m3 code of a row's
# requantisation falling on the other side of a rounding midpoint (the GPU's
# h differs from the oracle's by accumulation order and the SiLU's
# exp/reciprocal, up to ~6e-5 of the row maximum) moves a token by ~2e-2:
# measured 2.3e-2 (f = 128, token 33, one such code) and 2.2e-2 (f = 192,
# token 4), on the separate requantisation launch exactly as on the fused one
# (they agree bit for bit); 2.8e-5 with requantisation off.
TOKEN_CHECKED = ("f192-elastic", "f64-shared", "f192-ragged")


@pytest.fixture(scope="module", params=list(RQ_SPECS))
def rq(request):
    L = Layer(RQ_SPECS[request.param])
    L.key = request.param
    return L


def _forward(L: Layer, T: int, fused: bool, monkeypatch):
    monkeypatch.setenv("FP8MOE_RQ", "1" if fused else "0")
    spec = L.spec
    x = L.x[:T].contiguous()
    kpt = None if L.kpt is None else L.kpt[:T].contiguous()
    ids = torch.empty((T, spec.k), dtype=torch.int32, device=dev())
    out = L.layer().forward(x, k_per_token=kpt, topk_ids=ids)
    torch.cuda.synchronize()
    return out, ids


@pytest.mark.parametrize("msub", [0, 1, 2, 4, 8])
def test_fused_requant_bit_exact(rq, msub, monkeypatch):
    """Fused and separate requantisation give the same output bit for bit, at
    the planner's row-pass height and at every forced one, on the whole
    batch, one token and a ragged prefix."""
    if msub:
        monkeypatch.setenv("FP8MOE_MSUB", str(msub))
    for T in sorted({rq.spec.T, 1, max(1, rq.spec.T // 3)}):
        a, ia = _forward(rq, T, True, monkeypatch)
        b, ib = _forward(rq, T, False, monkeypatch)
        assert torch.equal(ia, ib)
        assert torch.equal(a, b), f"T={T}: max |diff| {(a - b).abs().max().item():.3e}"


def test_fused_requant_vs_oracle(rq, monkeypatch):
    monkeypatch.setenv("FP8MOE_RQ", "1")
    if rq.key in TOKEN_CHECKED:
        err, worst = _check(rq)
        print(f"{rq.key}: rel-L2 {err:.3e}, worst token {worst:.3e}")
        return
    spec = rq.spec
    x = rq.x.contiguous()
    logits = lib().router_logits(x, rq.w_router)
    ids = torch.empty((spec.T, spec.k), dtype=torch.int32, device=dev())
    out = rq.layer().forward(x, topk_ids=ids)
    torch.cuda.synchronize()
    ref, ido, _ = oracle.forward(to_np(x), rq.qw, spec.k, logits_override=to_np(logits))
    np.testing.assert_array_equal(to_np(ids), ido)
    err = rel_l2(to_np(out), ref)
    per = row_rel_l2(to_np(out), ref)
    print(f"{rq.key}: rel-L2 {err:.3e}, worst token {per.max():.3e} (token {int(per.argmax())})")
    assert err <= TOL_REQUANT


def test_fused_requant_prism_full_size(monkeypatch):
    """The MoE-Prism-shaped layer at its real batch (T = 1024, 512
    sub-experts of f = 192, per-token k in {4, 8, 16, 32}): fused and
    separate requantisation equal bit for bit (its oracle parity on every
    token is test_gpu_layer.py::test_prism_elastic_k)."""
    L = Layer(wl.PRISM, want_oracle=False)
    a, ia = _forward(L, wl.PRISM.T, True, monkeypatch)
    b, ib = _forward(L, wl.PRISM.T, False, monkeypatch)
    assert torch.equal(ia, ib)
    assert torch.equal(a, b), f"max |diff| {(a - b).abs().max().item():.3e}"
    assert np.isfinite(to_np(a)).all()


COMBINE_SPECS = {
    "prism-like": wl.TINY.with_(T=90, d=2048, f=192, E=64, k=32, k_choices=(4, 8, 16, 32)),
    "shared": wl.TINY.with_(T=40, d=256, f=192, E=8, k=2, n_shared=2),
    "ragged-d": wl.TINY.with_(T=33, d=320, f=512, E=16, k=6, n_shared=1),
}


@pytest.mark.parametrize("name", list(COMBINE_SPECS))
def test_combine_row_kernel_bit_exact(name, monkeypatch):
    """The one-slab combine (every slot lookup of a token at once, the valid
    slots' rows SL at a time) adds the same rows in the same order as the
    slot-group combine, so the layer output is the same bit for bit with
    either (FP8MOE_COMBINE_ROW_T=1: always the one-slab kernel; 10**9:
    never), with per-token k, shared experts and a ragged d."""
    L = Layer(COMBINE_SPECS[name], want_oracle=False)
    monkeypatch.setenv("FP8MOE_DOWN_SPLITS", "1")
    outs = []
    for row_t in ("1", str(10 ** 9)):
        monkeypatch.setenv("FP8MOE_COMBINE_ROW_T", row_t)
        outs.append(_forward(L, L.spec.T, True, monkeypatch)[0])
    assert torch.equal(outs[0], outs[1]), f"max |diff| {(outs[0] - outs[1]).abs().max().item():.3e}"
