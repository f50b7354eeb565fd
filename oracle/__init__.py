"""CPU oracle for the W8A8 FP8 MoE layer -- TEST INFRASTRUCTURE ONLY.

The plain, slow definition of the layer (router -> top-k ids and weights ->
only the selected expert FFNs -> weighted sum restored to token order, as in
the blog post "Routage MoE entre GPU"; W8A8 FP8 as in the Alpha-MoE article's
opening section).  Implemented in plain C (moe_oracle.c) with fp32
accumulation in a fixed order; this module only marshals numpy arrays.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it.  It shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes as C
import pathlib
from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import build as _build

_LIB: Optional[C.CDLL] = None
F_NO_REQUANT = 1

_f32p = C.POINTER(C.c_float)
_i32p = C.POINTER(C.c_int32)
_u8p = C.POINTER(C.c_uint8)


class _Dims(C.Structure):
    _fields_ = [("T", C.c_int32), ("d", C.c_int32), ("f", C.c_int32), ("E", C.c_int32),
                ("k_max", C.c_int32), ("n_shared", C.c_int32), ("block_m", C.c_int32),
                ("flags", C.c_uint32)]


class _Weights(C.Structure):
    _fields_ = [("w_gate", _u8p), ("w_up", _u8p), ("s_gate", _f32p), ("s_up", _f32p),
                ("w_down", _u8p), ("s_down", _f32p),
                ("ws_gate", _u8p), ("ws_up", _u8p), ("ws_down", _u8p),
                ("ss_gate", _f32p), ("ss_up", _f32p), ("ss_down", _f32p)]


def lib() -> C.CDLL:
    """Load the oracle library, building it only when it is not built yet."""
    global _LIB
    if _LIB is None:
        path = _build.LIB
        if not path.exists():
            _build.build()
        L = C.CDLL(str(path))
        L.moe_oracle_e4m3_encode.restype = C.c_uint8
        L.moe_oracle_e4m3_encode.argtypes = [C.c_float]
        L.moe_oracle_e4m3_decode.restype = C.c_float
        L.moe_oracle_e4m3_decode.argtypes = [C.c_uint8]
        L.moe_oracle_codec_selfcheck.restype = C.c_int64
        L.moe_oracle_codec_selfcheck.argtypes = [C.c_uint64, C.c_uint64, C.POINTER(C.c_uint32), C.c_int]
        L.moe_oracle_capacity.restype = C.c_int64
        L.moe_oracle_capacity.argtypes = [C.c_int32] * 4
        for name in ["e4m3_encode_array", "e4m3_decode_array"]:
            getattr(L, "moe_oracle_" + name).restype = None
        _LIB = L
    return _LIB


def _p(a: Optional[np.ndarray], ty):
    if a is None:
        return C.cast(None, ty)
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ty)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


# --------------------------------------------------------------------------- codec

def encode(v) -> np.ndarray:
    """e4m3 codes of fp32 values (nearest, ties to even code, saturating)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().moe_oracle_e4m3_encode_array(_p(v, _f32p), C.c_int64(v.size), _p(out, _u8p))
    return out


def decode(c) -> np.ndarray:
    """Exact fp32 value of e4m3 codes."""
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, dtype=np.float32)
    lib().moe_oracle_e4m3_decode_array(_p(c, _u8p), C.c_int64(c.size), _p(out, _f32p))
    return out


def codec_selfcheck(lo: int = 0, hi: int = 1 << 32, nthreads: int = 0):
    """(mismatches, first bad fp32 pattern) of the bit encoder against the
    nearest-value search, over fp32 patterns [lo, hi)."""
    first = C.c_uint32(0)
    bad = lib().moe_oracle_codec_selfcheck(lo, hi, C.byref(first), nthreads)
    return int(bad), int(first.value)


# --------------------------------------------------------------------------- weights

@dataclass
class QuantWeights:
    """e4m3 expert weights with fp32 per-output-channel scales (host arrays)."""
    w_gate: np.ndarray  # [E, f, d] uint8
    w_up: np.ndarray
    s_gate: np.ndarray  # [E, f] float32
    s_up: np.ndarray
    w_down: np.ndarray  # [E, d, f] uint8
    s_down: np.ndarray  # [E, d]
    ws_gate: Optional[np.ndarray] = None  # shared experts, same layouts
    ws_up: Optional[np.ndarray] = None
    ss_gate: Optional[np.ndarray] = None
    ss_up: Optional[np.ndarray] = None
    ws_down: Optional[np.ndarray] = None
    ss_down: Optional[np.ndarray] = None

    @property
    def n_shared(self) -> int:
        return 0 if self.ws_gate is None else int(self.ws_gate.shape[0])

    def _struct(self) -> _Weights:
        return _Weights(_p(self.w_gate, _u8p), _p(self.w_up, _u8p), _p(self.s_gate, _f32p),
                        _p(self.s_up, _f32p), _p(self.w_down, _u8p), _p(self.s_down, _f32p),
                        _p(self.ws_gate, _u8p), _p(self.ws_up, _u8p), _p(self.ws_down, _u8p),
                        _p(self.ss_gate, _f32p), _p(self.ss_up, _f32p), _p(self.ss_down, _f32p))


def quantize_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row e4m3 quantisation over the last axis: (codes, fp32 scale per row)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    cols = x.shape[-1]
    rows = x.size // cols
    q = np.empty(x.shape, dtype=np.uint8)
    s = np.empty(x.shape[:-1], dtype=np.float32)
    _check(lib().moe_oracle_quantize_rows(_p(x, _f32p), C.c_int32(rows), C.c_int32(cols),
                                          _p(q, _u8p), _p(s, _f32p)), "quantize_rows")
    return q, s


def quantize_weights(w_gate, w_up, w_down, ws_gate=None, ws_up=None, ws_down=None) -> QuantWeights:
    """Quantise fp32 expert weights per output channel ([.., f, d] rows over d,
    [.., d, f] rows over f)."""
    qg, sg = quantize_rows(w_gate)
    qu, su = quantize_rows(w_up)
    qd, sd = quantize_rows(w_down)
    qw = QuantWeights(qg, qu, sg, su, qd, sd)
    if ws_gate is not None:
        qw.ws_gate, qw.ss_gate = quantize_rows(ws_gate)
        qw.ws_up, qw.ss_up = quantize_rows(ws_up)
        qw.ws_down, qw.ss_down = quantize_rows(ws_down)
    return qw


# --------------------------------------------------------------------------- steps

def capacity(T: int, E: int, k_max: int, block_m: int) -> int:
    return int(lib().moe_oracle_capacity(T, E, k_max, block_m))


def router_logits(x, w_router, bias=None, nthreads: int = 0) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    w_router = np.ascontiguousarray(w_router, dtype=np.float32)
    bias = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    T, d = x.shape
    E = w_router.shape[0]
    out = np.empty((T, E), dtype=np.float32)
    _check(lib().moe_oracle_router_logits(_p(x, _f32p), _p(w_router, _f32p), _p(bias, _f32p),
                                          C.c_int32(T), C.c_int32(d), C.c_int32(E),
                                          _p(out, _f32p), C.c_int(nthreads)), "router_logits")
    return out


def route_topk(logits, k_max: int, k_per_token=None) -> tuple[np.ndarray, np.ndarray]:
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    kpt = None if k_per_token is None else np.ascontiguousarray(k_per_token, dtype=np.int32)
    ids = np.empty((T, k_max), dtype=np.int32)
    w = np.empty((T, k_max), dtype=np.float32)
    _check(lib().moe_oracle_route_topk(_p(logits, _f32p), C.c_int32(T), C.c_int32(E),
                                       C.c_int32(k_max), _p(kpt, _i32p), _p(ids, _i32p),
                                       _p(w, _f32p)), "route_topk")
    return ids, w


def permute(topk_ids, E: int, block_m: int, cap: Optional[int] = None) -> dict:
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    T, K = ids.shape
    cap = capacity(T, E, K, block_m) if cap is None else cap
    nbc = (cap + block_m - 1) // block_m
    out = dict(sorted_pairs=np.empty(cap, np.int32), expert_offsets=np.empty(E + 1, np.int32),
               block_expert=np.empty(nbc, np.int32), inv_pairs=np.empty(T * K, np.int32),
               n_blocks=np.empty(1, np.int32))
    _check(lib().moe_oracle_permute(_p(ids, _i32p), C.c_int32(T), C.c_int32(E), C.c_int32(K),
                                    C.c_int32(block_m), C.c_int32(cap),
                                    _p(out["sorted_pairs"], _i32p), _p(out["expert_offsets"], _i32p),
                                    _p(out["block_expert"], _i32p), _p(out["inv_pairs"], _i32p),
                                    _p(out["n_blocks"], _i32p)), "permute")
    out["capacity"] = cap
    return out


def _dims(T, d, f, E, k_max, n_shared, block_m, flags) -> _Dims:
    return _Dims(T, d, f, E, k_max, n_shared, block_m, flags)


def expert_gate_up(xq, sx, perm: dict, w: QuantWeights, E: int, k_max: int, block_m: int,
                   nthreads: int = 0) -> np.ndarray:
    """h[rows, f] in the stage row layout (routed padded rows, then shared)."""
    xq = np.ascontiguousarray(xq, dtype=np.uint8)
    sx = np.ascontiguousarray(sx, dtype=np.float32)
    T, d = xq.shape
    f = w.w_gate.shape[1]
    cap = perm["capacity"]
    rows = cap + w.n_shared * T
    h = np.zeros((rows, f), dtype=np.float32)
    dm = _dims(T, d, f, E, k_max, w.n_shared, block_m, 0)
    ws = w._struct()
    _check(lib().moe_oracle_expert_gate_up(C.byref(dm), C.c_int32(cap), _p(xq, _u8p),
                                           _p(sx, _f32p), _p(perm["sorted_pairs"], _i32p),
                                           _p(perm["expert_offsets"], _i32p), C.byref(ws),
                                           _p(h, _f32p), C.c_int(nthreads)), "expert_gate_up")
    return h


def expert_down(hq, sh, h, perm: dict, w: QuantWeights, T: int, E: int, k_max: int,
                block_m: int, no_requant: bool = False, nthreads: int = 0) -> np.ndarray:
    f = w.w_gate.shape[1]
    d = w.w_down.shape[1]
    cap = perm["capacity"]
    rows = cap + w.n_shared * T
    y = np.zeros((rows, d), dtype=np.float32)
    hq = None if hq is None else np.ascontiguousarray(hq, dtype=np.uint8)
    sh = None if sh is None else np.ascontiguousarray(sh, dtype=np.float32)
    h = None if h is None else np.ascontiguousarray(h, dtype=np.float32)
    dm = _dims(T, d, f, E, k_max, w.n_shared, block_m, F_NO_REQUANT if no_requant else 0)
    ws = w._struct()
    _check(lib().moe_oracle_expert_down(C.byref(dm), C.c_int32(cap), _p(hq, _u8p), _p(sh, _f32p),
                                        _p(h, _f32p), _p(perm["sorted_pairs"], _i32p),
                                        _p(perm["expert_offsets"], _i32p), C.byref(ws),
                                        _p(y, _f32p), C.c_int(nthreads)), "expert_down")
    return y


def combine(y, topk_ids, topk_w, perm: dict, T: int, d: int, E: int, n_shared: int,
            block_m: int) -> np.ndarray:
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    w = np.ascontiguousarray(topk_w, dtype=np.float32)
    y = np.ascontiguousarray(y, dtype=np.float32)
    K = ids.shape[1]
    out = np.empty((T, d), dtype=np.float32)
    dm = _dims(T, d, 1, E, K, n_shared, block_m, 0)
    _check(lib().moe_oracle_combine(C.byref(dm), C.c_int32(perm["capacity"]), _p(y, _f32p),
                                    _p(ids, _i32p), _p(w, _f32p), _p(perm["inv_pairs"], _i32p),
                                    _p(out, _f32p)), "combine")
    return out


def forward(x, w: QuantWeights, k_max: int, w_router=None, router_bias=None, k_per_token=None,
            logits_override=None, no_requant: bool = False, block_m: int = 16,
            nthreads: int = 0):
    """The whole layer token by token.  Returns (out [T,d], ids [T,k_max], w [T,k_max])."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    T, d = x.shape
    E, f = w.w_gate.shape[0], w.w_gate.shape[1]
    wr = None if w_router is None else np.ascontiguousarray(w_router, dtype=np.float32)
    b = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
    kpt = None if k_per_token is None else np.ascontiguousarray(k_per_token, dtype=np.int32)
    lo = None if logits_override is None else np.ascontiguousarray(logits_override, dtype=np.float32)
    out = np.empty((T, d), dtype=np.float32)
    ids = np.empty((T, k_max), dtype=np.int32)
    tw = np.empty((T, k_max), dtype=np.float32)
    dm = _dims(T, d, f, E, k_max, w.n_shared, block_m, F_NO_REQUANT if no_requant else 0)
    ws = w._struct()
    _check(lib().moe_oracle_forward(C.byref(dm), _p(x, _f32p), _p(wr, _f32p), _p(b, _f32p),
                                    _p(kpt, _i32p), C.byref(ws), _p(lo, _f32p), _p(out, _f32p),
                                    _p(ids, _i32p), _p(tw, _f32p), C.c_int(nthreads)), "forward")
    return out, ids, tw


def libpath() -> pathlib.Path:
    return _build.LIB
