"""Oracle self-checks (CPU only): the sparse, token-by-token oracle against the
dense "run every expert, mask by top-k" NumPy formulation, and the oracle's
stage functions composed against its own whole-layer forward."""
import numpy as np
import pytest

import oracle
import dense_ref
import workloads as wl


def _layer(spec, seed=0):
    ri = wl.routing_inputs(spec, seed)
    w = wl.expert_weights(spec, seed)
    np_ = lambda t: None if t is None else t.numpy()
    qw = oracle.quantize_weights(np_(w.w_gate), np_(w.w_up), np_(w.w_down),
                                 np_(w.ws_gate), np_(w.ws_up), np_(w.ws_down))
    dq = dense_ref.quantize_weights(np_(w.w_gate), np_(w.w_up), np_(w.w_down),
                                    np_(w.ws_gate), np_(w.ws_up), np_(w.ws_down))
    return ri, qw, dq


SMALL = [
    wl.TINY,
    wl.TINY.with_(name="t-shared", T=9, d=128, f=64, E=6, k=3, n_shared=2),
    wl.TINY.with_(name="t-elastic", T=20, d=64, f=192, E=16, k=8, k_choices=(1, 2, 4, 8)),
    wl.TINY.with_(name="t-one", T=1, d=64, f=64, E=4, k=1),
    wl.TINY.with_(name="t-zipf", T=24, d=128, f=128, E=32, k=4, bias="zipf", bias_param=1.0),
]


@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s.name)
@pytest.mark.parametrize("no_requant", [False, True])
def test_sparse_oracle_matches_dense_bruteforce(spec, no_requant):
    ri, qw, dq = _layer(spec)
    x = ri.x.numpy()
    wr = ri.w_router.numpy()
    b = None if ri.router_bias is None else ri.router_bias.numpy()
    kpt = None if ri.k_per_token is None else ri.k_per_token.numpy()
    out, ids, w = oracle.forward(x, qw, spec.k, w_router=wr, router_bias=b, k_per_token=kpt,
                                 no_requant=no_requant)
    logits = oracle.router_logits(x, wr, b)
    ref, ids2, w2 = dense_ref.dense_forward(x, wr, b, dq, spec.k, kpt, logits=logits,
                                            no_requant=no_requant)
    np.testing.assert_array_equal(ids, ids2)
    assert np.abs(w - w2).max() < 1e-6
    err = dense_ref.rel_l2(out, ref)
    # fp32 accumulation vs float64: 1e-6-level; with requant a code can flip
    # at an e4m3 rounding boundary when fp32 and float64 h differ in the last bit
    assert err < (1e-5 if not no_requant else 2e-6), err


@pytest.mark.parametrize("spec", SMALL[:3], ids=lambda s: s.name)
@pytest.mark.parametrize("no_requant", [False, True])
def test_stages_compose_to_forward_bit_exact(spec, no_requant):
    ri, qw, _ = _layer(spec)
    x = ri.x.numpy()
    wr = ri.w_router.numpy()
    kpt = None if ri.k_per_token is None else ri.k_per_token.numpy()
    bm = 16
    out, ids, w = oracle.forward(x, qw, spec.k, w_router=wr, k_per_token=kpt,
                                 no_requant=no_requant, block_m=bm)
    xq, sx = oracle.quantize_rows(x)
    logits = oracle.router_logits(x, wr)
    ids2, w2 = oracle.route_topk(logits, spec.k, kpt)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_array_equal(w, w2)
    perm = oracle.permute(ids2, spec.E, bm)
    h = oracle.expert_gate_up(xq, sx, perm, qw, spec.E, spec.k, bm)
    hq, sh = oracle.quantize_rows(h)
    y = oracle.expert_down(hq, sh, h, perm, qw, spec.T, spec.E, spec.k, bm, no_requant=no_requant)
    out2 = oracle.combine(y, ids2, w2, perm, spec.T, spec.d, spec.E, spec.n_shared, bm)
    np.testing.assert_array_equal(out, out2)


def test_unquantised_reference_distance_is_reported():
    """The quantised layer sits a few percent from the same layer in float64
    without any fp8 rounding (reported, documents the scale of fp8 error)."""
    spec = wl.TINY
    ri = wl.routing_inputs(spec)
    w = wl.expert_weights(spec)
    x = ri.x.numpy().astype(np.float64)
    qw = oracle.quantize_weights(w.w_gate.numpy(), w.w_up.numpy(), w.w_down.numpy())
    out, ids, tw = oracle.forward(ri.x.numpy(), qw, spec.k, w_router=ri.w_router.numpy())
    ref = np.zeros_like(x)
    for t in range(spec.T):
        for j in range(spec.k):
            e = ids[t, j]
            g = w.w_gate[e].numpy().astype(np.float64) @ x[t]
            u = w.w_up[e].numpy().astype(np.float64) @ x[t]
            h = g / (1 + np.exp(-g)) * u
            ref[t] += tw[t, j] * (w.w_down[e].numpy().astype(np.float64) @ h)
    err = dense_ref.rel_l2(out, ref)
    assert 1e-3 < err < 0.15, err
