"""End-to-end GPU parity of the fused layer (moe_fused_forward) against the
CPU oracle.

Routing is compared bit-exactly given identical logits (the oracle receives
the GPU router's logits as its override); outputs must be within rel-L2 2e-2
with fp8 requantisation of the SiLU*up intermediate and 1e-3 without, over
the whole batch AND for every token on its own (so one corrupted row, row
pass or work item cannot hide in the batch norm).  Every layer shape runs at
its real batch sizes, in the configuration the benchmark times, and every
token is compared.
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


def row_rel_l2(a, b) -> np.ndarray:
    """Relative L2 error of each row of a against b (float64)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b, axis=1)
    return np.linalg.norm(a - b, axis=1) / np.where(den > 0, den, 1.0)


def _check(L: Layer, T=None, no_requant=False, sample=None, block_m=16, seed=0, equal=False,
           persistent=False, bias=None, hot=None):
    """Run the GPU layer on the first T tokens; compare (a sample of) rows.
    bias: router bias replacing the layer's (device tensor); hot: (expert,
    tokens) the GPU routing must send to that expert."""
    spec = L.spec
    T = spec.T if T is None else T
    x = L.x[:T].contiguous()
    kpt = None if L.kpt is None else L.kpt[:T].contiguous()
    b = L.bias if bias is None else bias
    layer = lib().MoELayer(L.dw, L.w_router, spec.k, b, block_m, no_requant, persistent)
    m = lib()
    if equal:
        logits = torch.zeros((T, spec.E), dtype=torch.float32, device=dev())
    else:
        logits = m.router_logits(x, L.w_router, b)
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
    gids = to_np(ids)
    np.testing.assert_array_equal(gids[rows], ido)
    assert np.abs(to_np(w)[rows] - wo).max() < 2e-7
    if hot is not None:
        assert int((gids == hot[0]).sum()) == hot[1], "hot expert load"
    got = to_np(out)[rows]
    err = rel_l2(got, ref)
    per = row_rel_l2(got, ref)
    tol = TOL_NO_REQUANT if no_requant else TOL_REQUANT
    worst = int(np.argmax(per))
    assert err <= tol, f"rel-L2 {err:.3e} > {tol}"
    assert per[worst] <= tol, f"token {rows[worst]}: rel-L2 {per[worst]:.3e} > {tol}"
    return err, float(per[worst])


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
    err, worst = _check(small, no_requant=no_requant)
    print(f"{small.spec.name} no_requant={no_requant} rel-L2 {err:.3e} worst token {worst:.3e}")


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


@pytest.mark.parametrize("splits", [None, 1])
def test_deterministic_and_batch_invariant(small, splits, monkeypatch):
    """Repeated forwards are identical; a token's output does not depend on
    its batch (the ELDR page: outputs identical to standard top-k when only
    placement changes).  With one K split of the down projection (pinned) the
    batches differ only in rounding order, within 1e-6.  Left to the planner,
    the two batch sizes may take different split counts, and the fp16 y
    slabs then round different partial sums: each element within a few fp16
    half-ulps (2^-11 relative each), 2e-3 over the rows."""
    if splits is not None:
        monkeypatch.setenv("FP8MOE_DOWN_SPLITS", str(splits))
    layer = small.layer()
    kpt = small.kpt
    a = layer.forward(small.x, k_per_token=kpt)
    b = layer.forward(small.x, k_per_token=kpt)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    sub = torch.tensor([0, small.spec.T - 1], device=dev())
    c = layer.forward(small.x[sub].contiguous(), k_per_token=None if kpt is None else kpt[sub].contiguous())
    torch.cuda.synchronize()
    assert rel_l2(to_np(c), to_np(a)[to_np(sub)]) < (1e-6 if splits == 1 else 2e-3)


def _persistent_vs_staged(L: Layer, T=None, no_requant=False, bias=None):
    """The single launch against the per-stage launches: routing identical bit
    for bit, outputs within rounding of each other and within the oracle's
    bar, the launch deterministic, its status word 0."""
    spec = L.spec
    T = spec.T if T is None else T
    x = L.x[:T].contiguous()
    kpt = None if L.kpt is None else L.kpt[:T].contiguous()
    b = L.bias if bias is None else bias
    staged = lib().MoELayer(L.dw, L.w_router, spec.k, b, 16, no_requant, False)
    pers = lib().MoELayer(L.dw, L.w_router, spec.k, b, 16, no_requant, True)
    ids_a = torch.empty((T, spec.k), dtype=torch.int32, device=dev())
    ids_b = torch.full_like(ids_a, -7)
    w_a = torch.empty((T, spec.k), dtype=torch.float32, device=dev())
    w_b = torch.full_like(w_a, -7.0)
    a = staged.forward(x, k_per_token=kpt, topk_ids=ids_a, topk_w=w_a)
    p1 = pers.forward(x, k_per_token=kpt, topk_ids=ids_b, topk_w=w_b)
    torch.cuda.synchronize()
    assert pers.status() == 0, "a grid barrier timed out"
    p2 = pers.forward(x, k_per_token=kpt)
    torch.cuda.synchronize()
    assert pers.status() == 0, "a grid barrier timed out"
    assert torch.equal(ids_a, ids_b) and torch.equal(w_a, w_b)
    assert torch.equal(p1, p2), "single launch not deterministic"
    tol = TOL_NO_REQUANT if no_requant else TOL_REQUANT
    assert rel_l2(to_np(p1), to_np(a)) <= tol / 4
    lo = to_np(lib().router_logits(x, L.w_router, b))
    ref, ido, _ = oracle.forward(to_np(x), L.qw, spec.k, logits_override=lo,
                                 k_per_token=None if kpt is None else to_np(kpt),
                                 no_requant=no_requant)
    np.testing.assert_array_equal(to_np(ids_b), ido)
    err = rel_l2(to_np(p1), ref)
    per = row_rel_l2(to_np(p1), ref)
    assert err <= tol and per.max() <= tol, (err, per.max())
    return err, float(per.max())


@pytest.mark.parametrize("no_requant", [False, True])
def test_persistent_single_launch_matches_staged(small, no_requant):
    """One cooperative launch runs the stage device functions between grid
    barriers (the Alpha-MoE article's fused persistent kernel)."""
    err, worst = _persistent_vs_staged(small, no_requant=no_requant)
    for T in (1, 17):
        if T <= small.spec.T:
            _persistent_vs_staged(small, T=T, no_requant=no_requant)
    print(f"persistent {small.spec.name} no_requant={no_requant} rel-L2 {err:.3e} worst {worst:.3e}")


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


ARES_SPECS = {
    "ares-shared": wl.TINY.with_(T=40, d=1024, f=192, E=16, k=4, n_shared=1),
    "ares-tail": wl.TINY.with_(T=200, d=640, f=448, E=32, k=6, k_choices=(2, 4, 6)),
}


@pytest.mark.parametrize("name", list(ARES_SPECS))
@pytest.mark.parametrize("ntg", [2, 3, 8])
def test_a_resident_down_tiles(name, ntg, monkeypatch):
    """The down projection on A-resident tiles (the item's rows for the whole
    K range in LDS, several N-tiles per workgroup, weights prefetched across
    tile boundaries), forced onto small layers with a partial last tile, a
    64-byte K tail and shared experts: every token within the bar."""
    monkeypatch.setenv("FP8MOE_ARES_NTG", str(ntg))
    L = Layer(ARES_SPECS[name])
    err, worst = _check(L)
    for T in (1, 7):
        _check(L, T=T)
    print(f"{name} ntg={ntg} rel-L2 {err:.3e} worst token {worst:.3e}")


# ----------------------------------------------------------------- full-size layers, every token

def test_mixtral_decode_sweep():
    L = Layer(wl.MIXTRAL)
    for T in wl.MIXTRAL_DECODE_T:
        err, worst = _check(L, T=T)
        print(f"mixtral T={T} rel-L2 {err:.3e} worst token {worst:.3e}")
    _check(L, T=32, no_requant=True)
    _check(L, T=8, equal=True)


def test_qwen3_decode_and_prefill():
    L = Layer(wl.QWEN3.with_(T=4096, bias_param=0.0))
    err, worst = _check(L, T=4096)
    print(f"qwen3 T=4096 rel-L2 {err:.3e} worst token {worst:.3e}")
    err, worst = _check(L, T=64)
    print(f"qwen3 T=64 alpha=0 rel-L2 {err:.3e} worst token {worst:.3e}")
    # Zipf offsets calibrated for 16 .. 96 distinct experts in the T=64 batch
    for D in wl.QWEN3_D_TARGETS:
        spec = wl.QWEN3.with_(T=64, bias_param=wl.qwen3_alpha(D))
        b = wl.zipf_bias(spec, 0).to(dev())
        err, worst = _check(L, T=64, bias=b)
        ids = to_np(lib().route_topk(lib().router_logits(L.x[:64].contiguous(), L.w_router, b),
                                     spec.k)[0])
        assert len(np.unique(ids[ids >= 0])) == D
        print(f"qwen3 T=64 D={D} rel-L2 {err:.3e} worst token {worst:.3e}")


def test_deepseek_shared_and_hot_expert():
    """The hot expert receives 4x the mean load at every batch size (its
    bias calibrated per T on the oracle's routing), checked on the GPU's
    routing too; every token compared."""
    L = Layer(wl.DEEPSEEK.with_(T=wl.DEEPSEEK_T[-1], bias="none"))
    hot = wl.hot_expert_index(L.spec, 0)
    for T in wl.DEEPSEEK_T:
        b = wl.routing_inputs(wl.deepseek_spec(T).with_(T=1), 0).router_bias.to(dev())
        err, worst = _check(L, T=T, bias=b, hot=(hot, wl.deepseek_hot_target(T)))
        print(f"deepseek T={T} rel-L2 {err:.3e} worst token {worst:.3e}")
    b = wl.routing_inputs(wl.deepseek_spec(512).with_(T=1), 0).router_bias.to(dev())
    _check(L, T=512, bias=b, no_requant=True)


def test_prism_elastic_k():
    L = Layer(wl.PRISM)
    err, worst = _check(L)
    print(f"prism T=1024 rel-L2 {err:.3e} worst token {worst:.3e}")
    _check(L, no_requant=True)


def test_persistent_full_size():
    """The single launch at the real batch sizes: both row-pass kernels, the
    prefill tile, every routing regime (one wave per product, the routing
    tile with top-k inside, blocks of 128 experts), shared experts, elastic k."""
    L = Layer(wl.MIXTRAL)
    for T in (1, 32, 256):
        err, worst = _persistent_vs_staged(L, T=T)
        print(f"persistent mixtral T={T} rel-L2 {err:.3e} worst {worst:.3e}")
    del L
    L = Layer(wl.QWEN3.with_(T=4096, bias_param=0.0))
    for T in (64, 4096):
        err, worst = _persistent_vs_staged(L, T=T)
        print(f"persistent qwen3 T={T} rel-L2 {err:.3e} worst {worst:.3e}")
    del L
    L = Layer(wl.DEEPSEEK.with_(T=wl.DEEPSEEK_T[-1], bias="none"))
    for T in wl.DEEPSEEK_T:
        b = wl.routing_inputs(wl.deepseek_spec(T).with_(T=1), 0).router_bias.to(dev())
        err, worst = _persistent_vs_staged(L, T=T, bias=b)
        print(f"persistent deepseek T={T} rel-L2 {err:.3e} worst {worst:.3e}")
    del L
    L = Layer(wl.PRISM)
    err, worst = _persistent_vs_staged(L)
    print(f"persistent prism T=1024 rel-L2 {err:.3e} worst {worst:.3e}")
