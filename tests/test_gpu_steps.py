"""GPU parity of each step against the CPU oracle, through the C ABI.

Bit-exact: e4m3 codes and scales, top-k ids and slot order (given identical
logits), the permutation, and the expert products on integer-exact inputs.
Within tolerance: router logits, routing weights, h and y on random inputs.
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


# ----------------------------------------------------------------- codec

def test_e4m3_conversion_exhaustive_in_range():
    """Every fp32 bit pattern with |v| <= 448, both signs: rows [448, v...] have
    amax 448 so r = 1 and the GPU's codes are e4m3(v) itself; they must equal
    the oracle's encoder bit for bit."""
    m = lib()
    top = 0x43E00000  # bits of 448.0
    chunk = 1 << 26
    cols = 4096
    bad = 0
    for sign in (0, 0x80000000):
        for lo in range(0, top + 1, chunk):
            hi = min(top + 1, lo + chunk)
            bits = torch.arange(lo, hi, dtype=torch.int64, device=dev())
            n = bits.numel()
            pad = (-n) % (cols - 1)
            if pad:
                bits = torch.cat([bits, torch.zeros(pad, dtype=torch.int64, device=dev())])
            bits = (bits | sign).to(torch.int64)
            v = (bits.to(torch.int32) if sign == 0 else (bits - (1 << 32)).to(torch.int32)).view(torch.float32)
            rows = v.reshape(-1, cols - 1)
            x = torch.cat([torch.full((rows.shape[0], 1), 448.0, device=dev()), rows], dim=1).contiguous()
            q, s = m.quantize_rows(x)
            assert torch.all(s == 1.0)
            got = to_np(q[:, 1:].reshape(-1)[:n])
            want = oracle.encode(to_np(v[:n]))
            bad += int(np.count_nonzero(got != want))
            del bits, v, rows, x, q, s
    assert bad == 0


# ----------------------------------------------------------------- quantise / router

@pytest.mark.parametrize("rows,cols", [(1, 64), (37, 256), (300, 2048), (5, 14336)])
def test_quantize_rows_bit_exact(rows, cols):
    g = torch.Generator().manual_seed(rows * 7 + cols)
    x = torch.randn(rows, cols, generator=g) * 3
    x[0, :5] = 0.0
    if rows > 2:
        x[2] = 0.0
    q, s = lib().quantize_rows(x.to(dev()))
    qo, so = oracle.quantize_rows(x.numpy())
    np.testing.assert_array_equal(to_np(q), qo)
    np.testing.assert_array_equal(to_np(s), so)


@pytest.mark.parametrize("T,d,E,bias", [(1, 4096, 8, False), (37, 2048, 128, True),
                                        (100, 256, 8, False), (16, 2048, 512, True),
                                        (5, 64, 3, True),
                                        # more than 16 experts: K split over a workgroup's waves
                                        (512, 2048, 64, True), (19, 320, 200, False),
                                        # batches past the per-(token, expert) kernel: tiled fp32 MFMA path
                                        (1000, 320, 100, True), (4096, 2048, 128, False),
                                        (2100, 192, 32, True), (1100, 256, 64, True),
                                        # one K chunk (fewer than the prefetch depth), three
                                        # chunks, expert counts that pad the tile
                                        (1100, 64, 64, False), (3000, 192, 40, True),
                                        (3900, 128, 17, True), (2000, 320, 33, False),
                                        # two tokens x four experts per wave: odd T, E not a
                                        # multiple of 4, two 2048-float parts
                                        (301, 256, 70, True), (200, 4096, 100, False),
                                        # blocks of 128 experts (the last one ragged)
                                        (700, 256, 300, True), (1024, 2048, 512, True)])
def test_router_logits(T, d, E, bias):
    g = torch.Generator().manual_seed(T + d + E)
    x = torch.randn(T, d, generator=g)
    wr = torch.randn(E, d, generator=g) / d ** 0.5
    b = torch.randn(E, generator=g) if bias else None
    lg = lib().router_logits(x.to(dev()), wr.to(dev()), None if b is None else b.to(dev()))
    lo = oracle.router_logits(x.numpy(), wr.numpy(), None if b is None else b.numpy())
    err = np.abs(to_np(lg) - lo).max() / np.abs(lo).max()
    assert err < 1e-5, err


@pytest.mark.parametrize("T,E", [(3, 16), (300, 40), (3000, 40)])
def test_router_one_hot_exact(T, E):
    d = 256
    g = torch.Generator().manual_seed(3)
    wr = torch.randn(E, d, generator=g)
    b = torch.randn(E, generator=g)
    cols = torch.randint(0, d, (T,), generator=g)
    x = torch.zeros(T, d)
    x[torch.arange(T), cols] = 1.0
    lg = to_np(lib().router_logits(x.to(dev()), wr.to(dev()), b.to(dev())))
    np.testing.assert_array_equal(lg, (wr[:, cols].T + b).numpy())


@pytest.mark.parametrize("T,d,E,k,var", [(1100, 256, 64, 6, False), (700, 320, 100, 8, True),
                                         (2100, 192, 32, 4, True), (4096, 2048, 128, 8, False),
                                         (1100, 64, 64, 6, True), (3900, 128, 17, 17, False),
                                         (301, 256, 70, 6, True), (200, 4096, 100, 8, False),
                                         (700, 256, 300, 16, True)])
def test_prefill_routing_equals_steps(T, d, E, k, var):
    """Whichever routing kernels the batch size picks (the one-launch prefill
    routing for T*E > 65536 and E <= 128, the same tile over blocks of 128
    experts then a top-k launch for E > 128, two tokens x four experts per wave
    below 65536 pairs),
    the layer's ids and weights equal, bit for bit, those of moe_route_topk on
    moe_router_logits' logits, and the layer's output matches the oracle run
    on those logits."""
    m = lib()
    spec = wl.TINY.with_(T=T, d=d, f=128, E=E, k=k, bias="zipf", bias_param=1.0,
                         k_choices=tuple(range(1, k + 1)) if var else ())
    L = Layer(spec)
    kpt = L.kpt
    lg = m.router_logits(L.x, L.w_router, L.bias)
    ids_s, w_s = m.route_topk(lg, k, kpt)
    ids = torch.empty((T, k), dtype=torch.int32, device=dev())
    w = torch.empty((T, k), dtype=torch.float32, device=dev())
    out = L.layer().forward(L.x, k_per_token=kpt, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_s)
    assert torch.equal(w, w_s)
    rows = np.unique(np.random.default_rng(T).choice(T, min(T, 256), replace=False))
    ref, _, _ = oracle.forward(to_np(L.x)[rows], L.qw, k, logits_override=to_np(lg)[rows],
                               k_per_token=None if kpt is None else to_np(kpt)[rows])
    err = rel_l2(to_np(out)[rows], ref)
    assert err <= 2e-2, err


# ----------------------------------------------------------------- top-k

def _tie_logits(T, E, seed):
    rng = np.random.default_rng(seed)
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[0] = 0.25
    l[1, :] = np.where(rng.random(E) < 0.5, -0.0, 0.0)
    l[2] = np.round(l[2] * 2) / 2
    if T > 3:
        l[3, E // 2] = l[3, E // 3] = l[3].max() + 1
    return l


@pytest.mark.parametrize("T,E,k,var", [(16, 8, 2, False), (64, 128, 8, False), (31, 64, 6, False),
                                       (100, 512, 32, True), (7, 5, 5, False), (40, 32, 1, False),
                                       (1024, 512, 32, True),
                                       # just past one and two 64-expert slots per lane
                                       (33, 65, 7, False), (50, 200, 32, True)])
def test_topk_bit_exact(T, E, k, var):
    l = _tie_logits(T, E, T + E)
    kpt = None
    if var:
        kpt = np.random.default_rng(1).choice([4, 8, 16, 32], T).astype(np.int32)
    ids, w = lib().route_topk(torch.from_numpy(l).to(dev()), k,
                              None if kpt is None else torch.from_numpy(kpt).to(dev()))
    ido, wo = oracle.route_topk(l, k, kpt)
    np.testing.assert_array_equal(to_np(ids), ido)
    assert np.abs(to_np(w) - wo).max() < 2e-7
    s = to_np(w).astype(np.float64).sum(axis=1)
    kk = np.full(T, k) if kpt is None else kpt
    assert np.all(np.abs(s - 1.0) <= kk * 2.0 ** -23 + 1e-7)


# ----------------------------------------------------------------- permutation

@pytest.mark.parametrize("T,E,k,bm,var", [(16, 8, 2, 16, False), (1, 8, 2, 16, False),
                                          (256, 8, 2, 64, False), (64, 128, 8, 16, False),
                                          (1000, 512, 32, 32, True), (513, 64, 6, 1, False),
                                          (8192, 64, 6, 128, False), (3, 512, 4, 16, True),
                                          (2053, 64, 8, 16, False), (4096, 128, 8, 16, False),
                                          (5000, 512, 8, 1, True)])
@pytest.mark.parametrize("workspace", [False, True])
def test_permute_bit_exact(T, E, k, bm, var, workspace):
    """moe_permute, and moe_permute_ws (the two-launch form for batches of four
    or more 1024-pair slices: layout and scatter in one launch over the slice
    counts in the workspace), against the oracle, every array bit for bit."""
    rng = np.random.default_rng(T * 3 + E)
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[:, 0] += 2.0  # a hot expert
    kpt = rng.integers(1, k + 1, T).astype(np.int32) if var else None
    ids, _ = oracle.route_topk(l, k, kpt)
    p = lib().permute(torch.from_numpy(ids).to(dev()), E, bm, workspace=workspace)
    torch.cuda.synchronize()
    po = oracle.permute(ids, E, bm)
    for key in ("sorted_pairs", "expert_offsets", "block_expert", "inv_pairs", "n_blocks"):
        np.testing.assert_array_equal(to_np(p[key]), po[key], err_msg=key)


# ----------------------------------------------------------------- weight tile order

@pytest.mark.parametrize("R,C", [(16, 64), (48, 192), (64, 4096), (1408, 2048), (4096, 14336),
                                 (32, 16384)])
def test_pack_weights_bit_exact(R, C):
    """moe_pack_weights against the layout's definition (tests/tile_layout),
    including the zero padding of a 64-wide tail."""
    m = lib()
    rng = np.random.default_rng(R + C)
    codes = rng.integers(0, 256, (R, C), dtype=np.uint8)
    packed = m.pack_weights(torch.from_numpy(codes).to(dev()))
    assert packed.numel() == m.packed_weight_bytes(R, C)
    np.testing.assert_array_equal(to_np(packed), tl.pack(codes))


def test_pack_weights_rejects_bad_shapes():
    m = lib()
    codes = torch.zeros((24, 64), dtype=torch.uint8, device=dev())
    with pytest.raises(m.MoEError):
        m.pack_weights(codes, torch.empty(24 * 128, dtype=torch.uint8, device=dev()))
    assert m.packed_weight_bytes(24, 64) == 0 and m.packed_weight_bytes(16, 96) == 0


# ----------------------------------------------------------------- expert products

def _planted(rng, rows, cols, at, zero):
    """Small integers in [-4, 4]; column `at` holds +-448 (so amax = 448 and
    the scale is exactly 1) and column `zero` is 0."""
    a = rng.integers(-4, 5, (rows, cols)).astype(np.float32)
    a[:, at] = np.where(rng.random(rows) < 0.5, 448.0, -448.0)
    a[:, zero] = 0.0
    return a


@pytest.mark.parametrize("T,d,f,E,k,S", [(12, 256, 128, 4, 2, 0), (40, 320, 192, 8, 3, 1),
                                         (70, 256, 256, 2, 2, 0)])
def test_expert_products_integer_exact(T, d, f, E, k, S):
    """Integer operands whose +-448 entries (one column per side, which the
    other side zeroes) give scales of exactly 1 while every product stays a
    small integer: all partial sums are integers below 2^13, exact under any
    order or alignment of the MFMA's internal accumulation.  This pins the
    MFMA operand layouts, the K stepping (incl. the 64-wide tail), row
    gathering and the epilogue row/column mapping."""
    m = lib()
    rng = np.random.default_rng(T + d + f)
    x = _planted(rng, T, d, at=0, zero=1)
    wg = _planted(rng, (E + S) * f, d, at=1, zero=0).reshape(E + S, f, d)
    wu = _planted(rng, (E + S) * f, d, at=1, zero=0).reshape(E + S, f, d)
    wd = _planted(rng, (E + S) * d, f, at=1, zero=0).reshape(E + S, d, f)
    qw = oracle.quantize_weights(wg[:E], wu[:E], wd[:E], wg[E:] if S else None,
                                 wu[E:] if S else None, wd[E:] if S else None)
    dw = m.DeviceWeights.empty(E, d, f, S, device=dev())
    for e in range(E + S):
        sh = e >= E
        i = e - E if sh else e
        dw.set_expert("gate", i, torch.from_numpy(wg[e]).to(dev()), sh)
        dw.set_expert("up", i, torch.from_numpy(wu[e]).to(dev()), sh)
        dw.set_expert("down", i, torch.from_numpy(wd[e]).to(dev()), sh)
    np.testing.assert_array_equal(tl.unpack(to_np(dw.w_gate), f, d), qw.w_gate)
    np.testing.assert_array_equal(tl.unpack(to_np(dw.w_down), d, f), qw.w_down)
    ids, _ = oracle.route_topk(rng.standard_normal((T, E)).astype(np.float32), k)
    bm = 16
    perm_o = oracle.permute(ids, E, bm)
    perm = m.permute(torch.from_numpy(ids).to(dev()), E, bm)
    xq, sx = m.quantize_rows(torch.from_numpy(x).to(dev()))
    dm = m.dims(T, d, f, E, k, S, bm)
    h = to_np(m.expert_gate_up(dm, perm, xq, sx, dw))
    xqo, sxo = oracle.quantize_rows(x)
    ho = oracle.expert_gate_up(xqo, sxo, perm_o, qw, E, k, bm)
    real = np.ones(h.shape[0], bool)
    real[:perm_o["capacity"]] = perm_o["sorted_pairs"] != T * k
    # G and U are exact; only SiLU's exp may differ by an ulp between libm and the GPU
    np.testing.assert_allclose(h[real], ho[real], rtol=1e-6, atol=1e-30)
    # down projection on planted integer h codes: Y exact, y bit-exact
    hrows = _planted(rng, h.shape[0], f, at=0, zero=1)
    hq, sh = m.quantize_rows(torch.from_numpy(hrows).to(dev()))
    y = to_np(m.expert_down(dm, perm, dw, hq=hq, sh=sh))
    hqo, sho = oracle.quantize_rows(hrows)
    yo = oracle.expert_down(hqo, sho, None, perm_o, qw, T, E, k, bm)
    np.testing.assert_array_equal(y[real], yo[real])


@pytest.mark.parametrize("name", ["tiny", "shared", "elastic", "tall", "tall8"])
@pytest.mark.parametrize("no_requant", [False, True])
def test_expert_stages_random(name, no_requant, monkeypatch):
    spec = {"tiny": wl.TINY,
            "shared": wl.TINY.with_(T=33, d=256, f=192, E=6, k=3, n_shared=2),
            "elastic": wl.TINY.with_(T=50, d=128, f=320, E=32, k=8, k_choices=(1, 2, 4, 8)),
            # 256-row passes (prefill kernel): experts of about 300 rows and
            # a shared expert of 600 take two and three passes; K tails of 64
            # bytes (d = 704: 6 steps, f = 448: 4 steps); partial last
            # channel tiles
            "tall": wl.TINY.with_(T=600, d=704, f=448, E=4, k=2, n_shared=1),
            # 128-row passes: the down projection's K loop starts at a
            # rotated step per tile and wraps
            "tall8": wl.TINY.with_(T=600, d=704, f=448, E=4, k=2, n_shared=1)}[name]
    if name == "tall":
        monkeypatch.setenv("FP8MOE_MSUB", "16")
    if name == "tall8":
        monkeypatch.setenv("FP8MOE_MSUB", "8")
    m = lib()
    L = Layer(spec)
    bm = 16
    lo = oracle.router_logits(L.ri.x.numpy(), L.ri.w_router.numpy())
    kpt = None if L.ri.k_per_token is None else L.ri.k_per_token.numpy()
    ids, w = oracle.route_topk(lo, spec.k, kpt)
    perm_o = oracle.permute(ids, spec.E, bm)
    perm = m.permute(torch.from_numpy(ids).to(dev()), spec.E, bm)
    xq, sx = m.quantize_rows(L.x)
    dm = m.dims(spec.T, spec.d, spec.f, spec.E, spec.k, spec.n_shared, bm, no_requant)
    h = m.expert_gate_up(dm, perm, xq, sx, L.dw)
    xqo, sxo = oracle.quantize_rows(L.ri.x.numpy())
    ho = oracle.expert_gate_up(xqo, sxo, perm_o, L.qw, spec.E, spec.k, bm)
    real = np.ones(ho.shape[0], bool)
    real[:perm_o["capacity"]] = perm_o["sorted_pairs"] != spec.T * spec.k
    # The e4m3 MFMA does not round like a sequential fp32 sum: products that
    # span a wide exponent range lose low bits inside a K block (an order of
    # 1e-4 relative on one dot product, ~2e-5 rel-L2 measured on N(0,1) data),
    # so the stage bar is 1e-4 rather than fp32 rounding.
    err_h = rel_l2(to_np(h)[real], ho[real])
    print(f"{name} no_requant={no_requant}: h rel-L2 {err_h:.2e}")
    assert err_h < 1e-4
    # down from the oracle's own h (isolates the stage)
    if no_requant:
        y = m.expert_down(dm, perm, L.dw, h=torch.from_numpy(ho).to(dev()))
        yo = oracle.expert_down(None, None, ho, perm_o, L.qw, spec.T, spec.E, spec.k, bm, no_requant=True)
        tol = 1e-5  # fp32 products, fp32 accumulation
    else:
        hz = np.where(real[:, None], ho, 0).astype(np.float32)
        hqo, sho = oracle.quantize_rows(hz)
        y = m.expert_down(dm, perm, L.dw, hq=torch.from_numpy(hqo).to(dev()), sh=torch.from_numpy(sho).to(dev()))
        yo = oracle.expert_down(hqo, sho, None, perm_o, L.qw, spec.T, spec.E, spec.k, bm)
        tol = 1e-4  # e4m3 MFMA accumulation, as above
    err_y = rel_l2(to_np(y)[real], yo[real])
    print(f"{name} no_requant={no_requant}: y rel-L2 {err_y:.2e}")
    assert err_y < tol
    out = m.combine(dm, perm, y, torch.from_numpy(ids).to(dev()), torch.from_numpy(w).to(dev()))
    outo = oracle.combine(yo, ids, w, perm_o, spec.T, spec.d, spec.E, spec.n_shared, bm)
    assert rel_l2(to_np(out), outo) < tol
