"""Invariants of the layer checked on the oracle (CPU only).

- k = E with equal logits: every weight is 1/E and the output is the mean of
  all expert outputs (layer statement: weighted sum of the selected experts).
- A token's output does not depend on the batch it is in, and permuting
  tokens permutes outputs (ELDR article: outputs stay identical to standard
  top-k when only the serving placement changes).
- Shared experts add separably to the routed sum.
- Sub-expert decomposition (MoE-Prism, "Moteur de Refactorisation de
  Modele": an expert cut into disjoint neuron groups): selecting all N
  sub-experts with weight 1/N gives the parent expert's output / N.
"""
import numpy as np
import pytest

import oracle
import dense_ref
import workloads as wl


def _q(spec, seed=0):
    w = wl.expert_weights(spec, seed)
    n = lambda t: None if t is None else t.numpy()
    return oracle.quantize_weights(n(w.w_gate), n(w.w_up), n(w.w_down),
                                   n(w.ws_gate), n(w.ws_up), n(w.ws_down))


def _one_hot_logits(T, E, e):
    l = np.zeros((T, E), np.float32)
    l[:, e] = 1.0
    return l


@pytest.mark.parametrize("no_requant", [False, True])
def test_k_equals_E_uniform_is_mean_of_experts(no_requant):
    spec = wl.TINY.with_(T=6, d=128, f=128, E=8, k=8)
    x = wl.routing_inputs(spec).x.numpy()
    qw = _q(spec)
    out, ids, w = oracle.forward(x, qw, 8, logits_override=np.zeros((6, 8), np.float32),
                                 no_requant=no_requant)
    np.testing.assert_array_equal(w, np.float32(1 / 8))
    per = [oracle.forward(x, qw, 1, logits_override=_one_hot_logits(6, 8, e),
                          no_requant=no_requant)[0].astype(np.float64) for e in range(8)]
    mean = sum(per) / 8
    assert dense_ref.rel_l2(out, mean) < 1e-6


def test_batch_invariance_and_permutation_equivariance():
    spec = wl.TINY.with_(T=24, d=128, f=128, E=16, k=4, k_choices=(1, 2, 4))
    ri = wl.routing_inputs(spec)
    x, wr, kpt = ri.x.numpy(), ri.w_router.numpy(), ri.k_per_token.numpy()
    qw = _q(spec)
    out, ids, w = oracle.forward(x, qw, 4, w_router=wr, k_per_token=kpt)
    sub = np.array([3, 17, 0, 11])
    out_s, ids_s, _ = oracle.forward(x[sub], qw, 4, w_router=wr, k_per_token=kpt[sub])
    np.testing.assert_array_equal(out_s, out[sub])
    np.testing.assert_array_equal(ids_s, ids[sub])
    perm = np.random.default_rng(0).permutation(spec.T)
    out_p, _, _ = oracle.forward(x[perm], qw, 4, w_router=wr, k_per_token=kpt[perm])
    np.testing.assert_array_equal(out_p, out[perm])


def test_shared_experts_are_separable():
    spec = wl.TINY.with_(T=10, d=128, f=64, E=8, k=2, n_shared=2)
    ri = wl.routing_inputs(spec)
    x, wr = ri.x.numpy(), ri.w_router.numpy()
    qw = _q(spec)
    out, _, _ = oracle.forward(x, qw, 2, w_router=wr)
    routed = oracle.QuantWeights(qw.w_gate, qw.w_up, qw.s_gate, qw.s_up, qw.w_down, qw.s_down)
    out_r, _, _ = oracle.forward(x, routed, 2, w_router=wr)
    # each shared expert run as the only, weight-1 routed expert
    ys = 0
    for s in range(2):
        one = oracle.QuantWeights(qw.ws_gate[s:s + 1], qw.ws_up[s:s + 1], qw.ss_gate[s:s + 1],
                                  qw.ss_up[s:s + 1], qw.ws_down[s:s + 1], qw.ss_down[s:s + 1])
        ys = ys + oracle.forward(x, one, 1, logits_override=np.zeros((10, 1), np.float32))[0].astype(np.float64)
    assert dense_ref.rel_l2(out, out_r.astype(np.float64) + ys) < 1e-6
    # zero shared down-projection: exactly the routed-only output
    zero = oracle.QuantWeights(qw.w_gate, qw.w_up, qw.s_gate, qw.s_up, qw.w_down, qw.s_down,
                               qw.ws_gate, qw.ws_up, qw.ss_gate, qw.ss_up,
                               np.zeros_like(qw.ws_down), qw.ss_down)
    out_z, _, _ = oracle.forward(x, zero, 2, w_router=wr)
    np.testing.assert_array_equal(out_z, out_r)


@pytest.mark.parametrize("N", [2, 4])
def test_sub_expert_decomposition(N):
    spec = wl.TINY.with_(T=8, d=128, f=256, E=1, k=1)
    x = wl.routing_inputs(spec).x.numpy()
    qw = _q(spec)
    parent, _, _ = oracle.forward(x, qw, 1, logits_override=np.zeros((8, 1), np.float32),
                                  no_requant=True)
    c = spec.f // N
    # disjoint neuron groups: rows of W_gate/W_up, columns of W_down; codes and
    # per-channel scales carried over unchanged
    sub = oracle.QuantWeights(
        np.ascontiguousarray(qw.w_gate[0].reshape(N, c, spec.d)),
        np.ascontiguousarray(qw.w_up[0].reshape(N, c, spec.d)),
        np.ascontiguousarray(qw.s_gate[0].reshape(N, c)),
        np.ascontiguousarray(qw.s_up[0].reshape(N, c)),
        np.ascontiguousarray(qw.w_down[0].reshape(spec.d, N, c).transpose(1, 0, 2)),
        np.ascontiguousarray(np.broadcast_to(qw.s_down[0], (N, spec.d))))
    out, _, w = oracle.forward(x, sub, N, logits_override=np.zeros((8, N), np.float32),
                               no_requant=True)
    np.testing.assert_array_equal(w, np.float32(1 / N))
    assert dense_ref.rel_l2(out, parent.astype(np.float64) / N) < 1e-6
