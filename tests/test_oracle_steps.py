"""Pins for each oracle step (CPU only): quantisation, router, top-k and
weights, permutation, and the expert products on integer-exact inputs."""
import numpy as np
import pytest

import oracle
import dense_ref


# ----------------------------------------------------------------- quantisation

def test_quantize_matches_independent_formulation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[3] = 0.0
    x[5, 7] = 1e-30
    q, s = oracle.quantize_rows(x)
    q2, s2 = dense_ref.quantize_rows(x)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s, s2)


def test_quantize_row_max_maps_to_448_and_zero_row():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 128)).astype(np.float32)
    x[1] = 0.0
    q, s = oracle.quantize_rows(x)
    for r in range(8):
        if r == 1:
            assert np.all(q[r] == 0) and s[r] == 1.0
            continue
        i = np.argmax(np.abs(x[r]))
        assert q[r, i] & 0x7F == 0x7E  # |max| -> 448
        assert s[r] == np.float32(np.abs(x[r]).max()) / np.float32(448)


@pytest.mark.parametrize("n", [-3, 1, 7])
def test_quantize_power_of_two_invariance(n):
    # scaling a row by 2^n leaves the codes unchanged and scales s by 2^n
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    q, s = oracle.quantize_rows(x)
    q2, s2 = oracle.quantize_rows(x * np.float32(2.0 ** n))
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(s2, s * np.float32(2.0 ** n))


def test_quantize_dequant_error_bound():
    # |x - dec(q)*s| <= half an e4m3 ulp of the scaled value, relative 2^-4 (normal range)
    rng = np.random.default_rng(4)
    x = rng.standard_normal((32, 512)).astype(np.float32)
    q, s = oracle.quantize_rows(x)
    xr = oracle.decode(q) * s[:, None]
    big = np.abs(x) * (448 / np.abs(x).max(axis=1, keepdims=True)) >= 2.0 ** -6
    err = np.abs(xr - x)[big] / np.abs(x)[big]
    assert err.max() <= 2.0 ** -4 + 1e-6


def test_quantize_rejects_nonfinite():
    x = np.ones((2, 8), np.float32)
    x[1, 3] = np.inf
    with pytest.raises(ValueError):
        oracle.quantize_rows(x)


# ----------------------------------------------------------------- router

def test_router_one_hot_is_exact_column():
    rng = np.random.default_rng(5)
    d, E = 64, 16
    wr = rng.standard_normal((E, d)).astype(np.float32)
    b = rng.standard_normal(E).astype(np.float32)
    x = np.eye(d, dtype=np.float32)[[0, 5, 63]]
    l = oracle.router_logits(x, wr, b)
    for r, i in enumerate([0, 5, 63]):
        np.testing.assert_array_equal(l[r], wr[:, i] + b)
    l0 = oracle.router_logits(x, wr, None)
    np.testing.assert_array_equal(l0[1], wr[:, 5])


def test_router_matches_float64():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((33, 512)).astype(np.float32)
    wr = (rng.standard_normal((24, 512)) / np.sqrt(512)).astype(np.float32)
    b = rng.standard_normal(24).astype(np.float32)
    l = oracle.router_logits(x, wr, b)
    ref = x.astype(np.float64) @ wr.astype(np.float64).T + b
    assert np.abs(l - ref).max() <= 1e-5 * np.abs(ref).max()


# ----------------------------------------------------------------- top-k + weights

def _brute_force_check(logits, ids, kpt):
    T, E = logits.shape
    for t in range(T):
        kt = kpt[t]
        sel = list(ids[t, :kt])
        assert all(i == -1 for i in ids[t, kt:])
        assert len(set(sel)) == kt
        # slot order: (logit desc, index asc)
        for a, b in zip(sel, sel[1:]):
            la, lb = logits[t, a], logits[t, b]
            assert la > lb or (la == lb and a < b)
        # every selected beats every unselected
        for u in range(E):
            if u in sel:
                continue
            last = sel[-1]
            assert logits[t, last] > logits[t, u] or (logits[t, last] == logits[t, u] and last < u)


@pytest.mark.parametrize("E,k", [(8, 2), (64, 6), (128, 8), (512, 32), (5, 5)])
def test_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 100 + k)
    T = 40
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[0, :] = 0.5                                   # all equal
    logits[1, 3] = logits[1, 1] = logits[1].max() + 1    # tie at the top
    logits[2, : E // 2] = np.round(logits[2, : E // 2])  # many ties
    ids, w = oracle.route_topk(logits, k)
    _brute_force_check(logits, ids, [k] * T)
    np.testing.assert_array_equal(ids[0], np.arange(k))
    assert ids[1, 0] == 1 and ids[1, 1] == 3


def test_topk_signed_zero_is_a_tie():
    logits = np.array([[-0.0, 0.0, -1.0, -0.0]], dtype=np.float32)
    ids, w = oracle.route_topk(logits, 3)
    np.testing.assert_array_equal(ids[0], [0, 1, 3])
    np.testing.assert_array_equal(w[0], np.float32(1) / np.float32(3))


def test_topk_k_equals_E_is_full_order():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((6, 16)).astype(np.float32)
    ids, _ = oracle.route_topk(logits, 16)
    want = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    np.testing.assert_array_equal(ids, want)


def test_topk_variable_k_is_prefix_and_renormalised():
    rng = np.random.default_rng(8)
    T, E = 50, 64
    logits = rng.standard_normal((T, E)).astype(np.float32)
    kpt = rng.choice([4, 8, 16, 32], T).astype(np.int32)
    ids, w = oracle.route_topk(logits, 32, kpt)
    full, _ = oracle.route_topk(logits, 32)
    _brute_force_check(logits, ids, kpt)
    for t in range(T):
        np.testing.assert_array_equal(ids[t, :kpt[t]], full[t, :kpt[t]])
        assert np.all(w[t, kpt[t]:] == 0)
        assert abs(float(w[t].sum(dtype=np.float64)) - 1.0) <= kpt[t] * 2.0 ** -23
    # matches the independent float64 routing within fp32 rounding
    ids2, w2 = dense_ref.route(logits, 32, kpt)
    np.testing.assert_array_equal(ids, ids2)
    assert np.abs(w - w2).max() < 1e-6


def test_weights_closed_forms():
    logits = np.array([[3.0, 1.0, 2.0, 0.0]], dtype=np.float32)
    ids, w = oracle.route_topk(logits, 1)
    assert ids[0, 0] == 0 and w[0, 0] == 1.0        # k=1 -> exactly 1
    for k in (2, 4):
        eq = np.zeros((1, 8), np.float32)
        _, w = oracle.route_topk(eq, k)
        np.testing.assert_array_equal(w[0], np.float32(1.0 / k))  # power-of-two k -> exact 1/k
    # two experts: w0 = 1 / (1 + e^-(l0-l1))
    _, w = oracle.route_topk(np.array([[1.5, 0.25]], np.float32), 2)
    assert abs(w[0, 0] - 1 / (1 + np.exp(-1.25))) < 1e-7


# ----------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,E,k,bm", [(16, 8, 2, 16), (100, 64, 6, 16), (37, 512, 32, 32),
                                      (5, 8, 2, 1), (1, 8, 2, 64), (300, 128, 8, 128)])
def test_permute_properties(T, E, k, bm):
    rng = np.random.default_rng(T * 7 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    kpt = rng.integers(1, k + 1, T).astype(np.int32) if T % 2 else None
    ids, _ = oracle.route_topk(logits, k, kpt)
    p = oracle.permute(ids, E, bm)
    sp, off, be, inv, nb = (p["sorted_pairs"], p["expert_offsets"], p["block_expert"],
                            p["inv_pairs"], int(p["n_blocks"][0]))
    P = T * k
    flat = ids.ravel()
    valid = np.nonzero(flat >= 0)[0]
    # counts = histogram, segments padded to multiples of bm
    cnt = np.bincount(flat[valid], minlength=E)
    seg = np.diff(off)
    assert np.all(seg % bm == 0) and np.all(seg >= cnt) and np.all(seg - cnt < bm)
    assert off[0] == 0 and nb * bm == off[-1]
    # real entries are a bijection onto the valid pairs; inverse composes to identity
    real = sp[sp != P]
    assert sorted(real.tolist()) == valid.tolist()
    np.testing.assert_array_equal(sp[inv[valid]], valid)
    assert np.all(inv[flat < 0] == -1)
    # equals a plain stable sort of the valid pairs by expert
    stable = valid[np.argsort(flat[valid], kind="stable")]
    np.testing.assert_array_equal(real, stable)
    # each segment: its pairs first, then sentinels; block map names the owner
    for e in range(E):
        s = sp[off[e]:off[e + 1]]
        assert np.all(flat[s[:cnt[e]]] == e) and np.all(s[cnt[e]:] == P)
        assert np.all(be[off[e] // bm: off[e + 1] // bm] == e)
    assert np.all(be[nb:] == -1) and np.all(sp[off[-1]:] == P)


def test_permute_empty_experts_get_no_blocks():
    ids = np.array([[3, 3], [3, -1]], dtype=np.int32)
    p = oracle.permute(ids, 8, 4)
    np.testing.assert_array_equal(p["expert_offsets"], [0, 0, 0, 0, 4, 4, 4, 4, 4])
    np.testing.assert_array_equal(p["sorted_pairs"][:4], [0, 1, 2, 4])
    np.testing.assert_array_equal(p["inv_pairs"], [0, 1, 2, -1])
    assert int(p["n_blocks"][0]) == 1


# ----------------------------------------------------------------- expert products

def _planted_int_rows(rng, rows, cols):
    """Small integers in [-4, 4] with one +-448 per row: amax 448, so r = s = 1
    and every code is exact."""
    a = rng.integers(-4, 5, (rows, cols)).astype(np.float32)
    j = rng.integers(0, cols, rows)
    a[np.arange(rows), j] = np.where(rng.random(rows) < 0.5, 448.0, -448.0)
    return a


def test_gate_up_and_down_integer_exact():
    """With integer operands every product and partial sum is an exact integer
    (< 2^24), so G, U and Y are exact whatever the order; checks orientation
    ([f][d] rows over d, [d][f] rows over f), gathering and the scale algebra."""
    rng = np.random.default_rng(9)
    T, d, f, E, k, bm = 12, 128, 64, 4, 2, 16
    x = _planted_int_rows(rng, T, d)
    wg = _planted_int_rows(rng, E * f, d).reshape(E, f, d)
    wu = _planted_int_rows(rng, E * f, d).reshape(E, f, d)
    wd = _planted_int_rows(rng, E * d, f).reshape(E, d, f)
    qw = oracle.quantize_weights(wg, wu, wd)
    for a in (qw.s_gate, qw.s_up, qw.s_down):
        assert np.all(a == 1.0)
    xq, sx = oracle.quantize_rows(x)
    assert np.all(sx == 1.0)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.route_topk(logits, k)
    perm = oracle.permute(ids, E, bm)
    h = oracle.expert_gate_up(xq, sx, perm, qw, E, k, bm)
    xi = x.astype(np.int64)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            r = perm["inv_pairs"][t * k + j]
            G = (wg[e].astype(np.int64) @ xi[t]).astype(np.float64)
            U = (wu[e].astype(np.int64) @ xi[t]).astype(np.float64)
            with np.errstate(over="ignore"):
                want = (G / (1 + np.exp(-G))) * U
            np.testing.assert_allclose(h[r], want, rtol=2e-6, atol=1e-30)
    # down projection on planted integer codes: Y exact
    hrows = _planted_int_rows(rng, h.shape[0], f)
    hq, sh = oracle.quantize_rows(hrows)
    y = oracle.expert_down(hq, sh, None, perm, qw, T, E, k, bm)
    for t in range(T):
        for j in range(k):
            e = ids[t, j]
            r = perm["inv_pairs"][t * k + j]
            want = wd[e].astype(np.int64) @ hrows[r].astype(np.int64)
            np.testing.assert_array_equal(y[r], want.astype(np.float32))
