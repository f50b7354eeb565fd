"""End-to-end GPU parity of the fused layer (moe_fused_forward) against the
CPU oracle.

Routing is compared bit-exactly given identical logits (the oracle receives
the GPU router's logits as its override); outputs must be within rel-L2 2e-2
with fp8 requantisation of the SiLU*up intermediate and 1e-3 without.  Small
layers are compared on every token; the full-size layers run at their real
batch sizes in the configuration the benchmark times, and the oracle
recomputes a sample of tokens one by one (tokens are independent given
their logits).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
import tile_layout as tl
from gpu_common import Layer, dev, lib, rel_l2, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

TOL_REQUANT = 2e-2
TOL_NO_REQUANT = 1e-3


def _check(L: Layer, T=None, no_requant=False, sample=None, block_m=16, seed=0, equal=False,
           persistent=False):
    """Run the GPU layer on the first T tokens; compare (a sample of) rows."""
    spec = L.spec
    T = spec.T if T is None else T
    x = L.x[:T].contiguous()
    kpt = None if L.kpt is None else L.kpt[:T].contiguous()
    layer = L.layer(block_m=block_m, no_requant=no_requant, persistent=persistent)
    m = lib()
    if equal:
        logits = torch.zeros((T, spec.E), dtype=torch.float32, device=dev())
    else:
        logits = m.router_logits(x, L.w_router, L.bias)
    ids = torch.empty((T, spec.k), dtype=torch.int32, device=dev())
    w = torch.empty((T, spec.k), dtype=torch.float32, device=dev())
    out = layer.forward(x, k_per_token=kpt, topk_ids=ids, topk_w=w,
                        logits_override=logits if equal else None)
    torch.cuda.synchronize()
    rows = np.arange(T) if sample is None else np.unique(
        np.random.default_rng(seed).choice(T, min(sample, T), replace=False))
    lo = to_np(logits)[rows]
    xs = to_np(x)[rows]
    ks = None if kpt is None else to_np(kpt)[rows]
    ref, ido, wo = oracle.forward(xs, L.qw, spec.k, logits_override=lo, k_per_token=ks,
                                  no_requant=no_requant, block_m=block_m)
    np.testing.assert_array_equal(to_np(ids)[rows], ido)
    assert np.abs(to_np(w)[rows] - wo).max() < 2e-7
    err = rel_l2(to_np(out)[rows], ref)
    tol = TOL_NO_REQUANT if no_requant else TOL_REQUANT
    assert err <= tol, f"rel-L2 {err:.3e} > {tol}"
    return err


# ----------------------------------------------------------------- small layers, every token

SMALL = {
    "tiny": wl.TINY,
    "tiny-shared": wl.TINY.with_(T=40, d=256, f=192, E=8, k=2, n_shared=2),
    "tiny-elastic": wl.TINY.with_(T=77, d=256, f=192, E=64, k=32, k_choices=(4, 8, 16, 32)),
    "tiny-zipf": wl.TINY.with_(T=64, d=512, f=256, E=128, k=8, bias="zipf", bias_param=2.0),
    "tiny-hot": wl.TINY.with_(T=96, d=256, f=1408 // 2, E=64, k=6, n_shared=2, bias="hot", bias_param=2.5),
    "ragged": wl.TINY.with_(T=19, d=320, f=448, E=5, k=3),
}


@pytest.fixture(scope="module", params=list(SMALL))
def small(request):
    return Layer(SMALL[request.param])


@pytest.mark.parametrize("no_requant", [False, True])
def test_small_layers_every_token(small, no_requant):
    err = _check(small, no_requant=no_requant)
    print(f"{small.spec.name} no_requant={no_requant} rel-L2 {err:.3e}")


@pytest.mark.parametrize("bm", [1, 32, 128])
def test_block_m_variants(small, bm):
    _check(small, block_m=bm)


def test_single_token_and_ragged_batches(small):
    for T in (1, 2, 17):
        if T <= small.spec.T:
            _check(small, T=T)


def test_equal_logits_tie_stress(small):
    # every logit equal: ids must be 0..k-1 for every token (lower index wins)
    _check(small, equal=True)


def test_weights_match_oracle_quantiser(small):
    sp = small.spec
    np.testing.assert_array_equal(tl.unpack(to_np(small.dw.w_gate), sp.f, sp.d), small.qw.w_gate)
    np.testing.assert_array_equal(tl.unpack(to_np(small.dw.w_down), sp.d, sp.f), small.qw.w_down)
    np.testing.assert_array_equal(to_np(small.dw.s_down), small.qw.s_down)


def test_deterministic_and_batch_invariant(small):
    layer = small.layer()
    kpt = small.kpt
    a = layer.forward(small.x, k_per_token=kpt)
    b = layer.forward(small.x, k_per_token=kpt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # a token's output does not depend on its batch (same kernels, same routing)
    sub = torch.tensor([0, small.spec.T - 1], device=dev())
    c = layer.forward(small.x[sub].contiguous(), k_per_token=None if kpt is None else kpt[sub].contiguous())
    torch.cuda.synchronize()
    assert rel_l2(to_np(c), to_np(a)[to_np(sub)]) < 1e-6


PERSISTENT_OFF = ("single-launch path switched off: its cooperative launch did not complete "
                  "on gfx950 under test (grid barrier never released); cause not established")


@pytest.mark.skip(reason=PERSISTENT_OFF)
def test_persistent_single_launch_matches_staged(small):
    """One cooperative launch runs the same stage functions as the seven
    per-stage kernels: outputs and routing must be bit-identical, and within
    the bar against the oracle."""
    _check(small, persistent=True)
    staged = small.layer()
    pers = small.layer(persistent=True)
    ids_a = torch.empty((small.spec.T, small.spec.k), dtype=torch.int32, device=dev())
    ids_b = torch.empty_like(ids_a)
    a = staged.forward(small.x, k_per_token=small.kpt, topk_ids=ids_a)
    b = pers.forward(small.x, k_per_token=small.kpt, topk_ids=ids_b)
    b2 = pers.forward(small.x, k_per_token=small.kpt)
    torch.cuda.synchronize()
    assert torch.equal(ids_a, ids_b)
    assert torch.equal(a, b) and torch.equal(b, b2)


@pytest.mark.parametrize("msub,waves,nb", [(16, 0, 2), (16, 6, 2), (16, 3, 2), (8, 8, 2), (8, 7, 2),
                                           (2, 5, 2), (1, 1, 2), (8, 7, 4), (4, 5, 4), (2, 3, 4),
                                           (1, 6, 4)])
def test_gemm_geometry_overrides(small, msub, waves, nb, monkeypatch):
    """Every row-pass height, compute-wave count and operand count of the
    grouped GEMMs (tile-tuning overrides) gives the same parity, on every
    token.  msub 16 without a wave count runs the prefill kernel (eight
    waves that all gather and compute), with one the loader-wave kernel."""
    monkeypatch.setenv("FP8MOE_MSUB", str(msub))
    monkeypatch.setenv("FP8MOE_WAVES", str(waves))
    monkeypatch.setenv("FP8MOE_NB", str(nb))
    _check(small)
    _check(small, no_requant=True)


@pytest.mark.parametrize("msub,splits", [(16, 2), (16, 3), (4, 2), (4, 3)])
def test_down_k_splits(small, msub, splits, monkeypatch):
    """The down projection cut into K splits (partial sums in separate y
    slabs, added in split order by the combine), on the prefill kernel
    (msub 16) and a decode shape: the same parity on every token."""
    monkeypatch.setenv("FP8MOE_MSUB", str(msub))
    monkeypatch.setenv("FP8MOE_DOWN_SPLITS", str(splits))
    _check(small)


@pytest.mark.parametrize("ms,ml", [(1, 2), (1, 4), (1, 8), (2, 4), (2, 8), (4, 8)])
def test_two_shape_gemm(small, ms, ml, monkeypatch):
    """Work items cut at 16*ml rows, the ones of at most 16*ms rows on the
    short row-pass shape and the rest on the long one, in one launch: the
    same parity on every token."""
    monkeypatch.setenv("FP8MOE_MSUB", str(ms))
    monkeypatch.setenv("FP8MOE_MSUB_BIG", str(ml))
    _check(small)
    _check(small, no_requant=True)
    _check(small, block_m=32)


@pytest.mark.parametrize("nt", [0, 1])
def test_streamed_weight_loads(small, nt, monkeypatch):
    """The grouped GEMMs with and without the non-temporal weight-load hint
    give the same parity on every token."""
    monkeypatch.setenv("FP8MOE_NT", str(nt))
    _check(small)
    _check(small, no_requant=True)


def test_persistent_flag_is_refused(small):
    for nr in (False, True):
        with pytest.raises(lib().MoEError):
            small.layer(no_requant=nr, persistent=True).forward(small.x, k_per_token=small.kpt)


# ----------------------------------------------------------------- full-size layers, sampled

def test_mixtral_decode_sweep():
    L = Layer(wl.MIXTRAL)
    for T in wl.MIXTRAL_DECODE_T:
        err = _check(L, T=T, sample=6, seed=T)
        print(f"mixtral T={T} rel-L2 {err:.3e}")
    _check(L, T=32, sample=4, no_requant=True)
    _check(L, T=8, sample=4, equal=True)


def test_qwen3_decode_and_prefill():
    for alpha in (0.0, 1.5, 4.0):
        L = Layer(wl.QWEN3.with_(T=4096, bias_param=alpha))
        err = _check(L, T=64, sample=8, seed=1)
        print(f"qwen3 T=64 alpha={alpha} rel-L2 {err:.3e}")
        if alpha == 0.0:
            err = _check(L, T=4096, sample=8, seed=2)
            print(f"qwen3 T=4096 rel-L2 {err:.3e}")
        del L


def test_deepseek_shared_and_hot_expert():
    L = Layer(wl.DEEPSEEK.with_(T=8192, bias_param=2.0))
    for T in wl.DEEPSEEK_T:
        err = _check(L, T=T, sample=6, seed=T)
        print(f"deepseek T={T} rel-L2 {err:.3e}")


def test_prism_elastic_k():
    L = Layer(wl.PRISM)
    err = _check(L, sample=8, seed=3)
    print(f"prism T=1024 rel-L2 {err:.3e}")
    _check(L, sample=4, seed=4, no_requant=True)


@pytest.mark.skip(reason=PERSISTENT_OFF)
def test_persistent_full_size():
    L = Layer(wl.MIXTRAL)
    for T in (1, 256):
        _check(L, T=T, sample=4, seed=T + 1, persistent=True)
    del L
    L = Layer(wl.QWEN3.with_(T=4096))
    _check(L, T=4096, sample=4, seed=5, persistent=True)
    del L
    L = Layer(wl.PRISM)
    _check(L, sample=4, seed=6, persistent=True)
