"""Dense brute-force formulation of the MoE layer, used to pin the oracle.

"Run every expert on every token, then mask by the top-k routing weights":
written with NumPy in float64 from the layer's definition, sharing nothing
with the C oracle (its own e4m3 table and nearest-value encoder, its own
routing by a stable argsort, its own dense expert products).  Where a
floating-point value decides an e4m3 code (x * r, h * r) it is taken in fp32,
the precision the oracle and the kernels use for that decision.
"""
from __future__ import annotations

import numpy as np


def e4m3_values() -> np.ndarray:
    """Value of every e4m3 (E4M3FN) code from the format definition."""
    c = np.arange(256)
    s, e, m = c >> 7, (c >> 3) & 15, c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return np.where(s == 1, -v, v)


_VALS = e4m3_values()
_POS = _VALS[:127]  # codes 0x00..0x7E: increasing, finite


def encode_nearest(v) -> np.ndarray:
    """Nearest finite e4m3 value (ties to the even code), sign copied, NaN -> 0x7F."""
    v = np.asarray(v, dtype=np.float32)
    av = np.abs(v.astype(np.float64))
    lo = np.clip(np.searchsorted(_POS, av, side="right") - 1, 0, 126)
    hi = np.minimum(lo + 1, 126)
    dlo = av - _POS[lo]
    dhi = _POS[hi] - av
    pick_hi = (hi != lo) & ((dhi < dlo) | ((dhi == dlo) & (lo % 2 == 1)))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(av >= 448.0, 0x7E, code).astype(np.uint8)
    code = code | np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return np.where(np.isnan(v), 0x7F, code).astype(np.uint8)


def decode(c) -> np.ndarray:
    return _VALS[np.asarray(c, dtype=np.uint8)]


def quantize_rows(x):
    """Per-row scale s = amax/448, codes of fp32(x * fp32(448/amax))."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), amax).astype(np.float32)
    r = np.where(zero, np.float32(1), np.float32(448.0) / safe).astype(np.float32)
    s = np.where(zero, np.float32(1), safe / np.float32(448.0)).astype(np.float32)
    q = encode_nearest((x * r[..., None]).astype(np.float32))
    return q, s


def route(logits, k_max, k_per_token=None):
    """ids/weights: stable descending sort (ties keep the lower index),
    softmax over each token's own k in float64."""
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    ids = np.full((T, k_max), -1, dtype=np.int64)
    w = np.zeros((T, k_max), dtype=np.float64)
    for t in range(T):
        kt = k_max if k_per_token is None else int(k_per_token[t])
        sel = order[t, :kt]
        l = logits[t, sel].astype(np.float64)
        ex = np.exp(l - l[0])
        ids[t, :kt] = sel
        w[t, :kt] = ex / ex.sum()
    return ids, w


def dense_forward(x, w_router, router_bias, wq: dict, k_max, k_per_token=None, logits=None,
                  no_requant=False):
    """wq: dict of e4m3 codes/scales (w_gate, s_gate, w_up, s_up, w_down,
    s_down, optional ws_*/ss_* for shared experts).  Returns (out, ids, w)."""
    x = np.asarray(x, dtype=np.float32)
    T, d = x.shape
    E = wq["w_gate"].shape[0]
    if logits is None:
        logits = (x.astype(np.float64) @ np.asarray(w_router, np.float64).T)
        if router_bias is not None:
            logits = logits + np.asarray(router_bias, np.float64)
        logits = logits.astype(np.float32)
    ids, w = route(logits, k_max, k_per_token)
    mask = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for j in range(k_max):
            if ids[t, j] >= 0:
                mask[t, ids[t, j]] = w[t, j]
    xq, sx = quantize_rows(x)
    xv = decode(xq) * sx.astype(np.float64)[:, None]

    def run_expert(wg, sg, wu, su, wd, sd):
        g = (xv @ decode(wg).T) * sg.astype(np.float64)[None, :]
        u = (xv @ decode(wu).T) * su.astype(np.float64)[None, :]
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        if no_requant:
            a = h.astype(np.float64)
        else:
            hq, sh = quantize_rows(h)
            a = decode(hq) * sh.astype(np.float64)[:, None]
        return (a @ decode(wd).T) * sd.astype(np.float64)[None, :]

    out = np.zeros((T, d), dtype=np.float64)
    for e in range(E):
        y = run_expert(wq["w_gate"][e], wq["s_gate"][e], wq["w_up"][e], wq["s_up"][e],
                       wq["w_down"][e], wq["s_down"][e])
        out += mask[:, e:e + 1] * y
    if wq.get("ws_gate") is not None:
        for s in range(wq["ws_gate"].shape[0]):
            out += run_expert(wq["ws_gate"][s], wq["ss_gate"][s], wq["ws_up"][s], wq["ss_up"][s],
                              wq["ws_down"][s], wq["ss_down"][s])
    return out, ids, w


def quantize_weights(w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None) -> dict:
    out = {}
    out["w_gate"], out["s_gate"] = quantize_rows(w_gate)
    out["w_up"], out["s_up"] = quantize_rows(w_up)
    out["w_down"], out["s_down"] = quantize_rows(w_down)
    if ws_gate is not None:
        out["ws_gate"], out["ss_gate"] = quantize_rows(ws_gate)
        out["ws_up"], out["ss_up"] = quantize_rows(ws_up)
        out["ws_down"], out["ss_down"] = quantize_rows(ws_down)
    return out


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = np.linalg.norm(b.ravel())
    return float(np.linalg.norm((a - b).ravel()) / (den if den > 0 else 1.0))
