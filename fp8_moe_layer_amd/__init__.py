"""fp8_moe_layer_amd -- W8A8 FP8 Mixture-of-Experts layer forward for AMD MI355X.

Thin ctypes binding over the gfx950 HIP library ``libfp8moe.so`` (C ABI in
``include/fp8moe.h``).  Every step of the layer runs in the library's
kernels; this module only turns torch tensors into pointers and the current
torch stream into a hipStream_t.  There is no CPU path: importing the package
fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import pathlib
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = pathlib.Path(__file__).resolve().parent
LIB_PATH = _HERE / "libfp8moe.so"
DEBUG_LIB_PATH = _HERE / "libfp8moe_debug.so"  # device-checked build of the same sources

MOE_F_NO_REQUANT = 1
MOE_F_PERSISTENT = 2
MOE_F_FUSED_COMBINE = 4
MAX_EXPERTS = 512
MAX_K = 32

if not LIB_PATH.exists():
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python fp8_moe_layer_amd/build.py` first (there is no CPU fallback)")

_lib = C.CDLL(str(LIB_PATH))

_vp = C.c_void_p
_i32 = C.c_int32


class Dims(C.Structure):
    _fields_ = [("T", _i32), ("d", _i32), ("f", _i32), ("E", _i32), ("k_max", _i32),
                ("n_shared", _i32), ("block_m", _i32), ("flags", C.c_uint32)]


class _Weights(C.Structure):
    _fields_ = [(n, _vp) for n in ("w_gate", "w_up", "s_gate", "s_up", "w_down", "s_down",
                                   "ws_gate", "ws_up", "ws_down", "ss_gate", "ss_up", "ss_down")]


def _sig(name, restype, *argtypes):
    fn = getattr(_lib, name)
    fn.restype = restype
    fn.argtypes = list(argtypes)
    return fn


_DP = C.POINTER(Dims)
_WP = C.POINTER(_Weights)
_quantize_rows = _sig("moe_quantize_rows", _i32, _vp, _i32, _i32, _vp, _vp, _vp)
_packed_weight_bytes = _sig("moe_packed_weight_bytes", C.c_int64, _i32, _i32)
_pack_weights = _sig("moe_pack_weights", _i32, _vp, _i32, _i32, _vp, _vp)
_router_logits = _sig("moe_router_logits", _i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _vp)
_route_topk = _sig("moe_route_topk", _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp)
_capacity = _sig("moe_capacity", C.c_int64, _i32, _i32, _i32, _i32)
_permute = _sig("moe_permute", _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp)
_permute_ws_bytes = _sig("moe_permute_workspace_bytes", C.c_size_t, _i32, _i32, _i32)
_permute_ws = _sig("moe_permute_ws", _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                   _vp, _vp, C.c_size_t, _vp)
_gate_up = _sig("moe_expert_gate_up", _i32, _DP, _i32, _vp, _vp, _vp, _vp, _WP, _vp, _vp)
_down = _sig("moe_expert_down", _i32, _DP, _i32, _vp, _vp, _vp, _vp, _vp, _WP, _vp, _vp)
_combine = _sig("moe_combine", _i32, _DP, _i32, _vp, _vp, _vp, _vp, _vp, _vp)
_workspace_bytes = _sig("moe_workspace_bytes", C.c_size_t, _DP)
_fused_forward = _sig("moe_fused_forward", _i32, _DP, _vp, _vp, _vp, _vp, _WP, _vp, _vp, _vp, _vp,
                      _vp, C.c_size_t, _vp)
_status_str = _sig("moe_status_str", C.c_char_p, _i32)
_last_error = _sig("moe_last_error", C.c_char_p)
_abi_version = _sig("moe_abi_version", _i32)
_fused_forward_timed = _sig("moe_fused_forward_timed", _i32, _DP, _vp, _vp, _vp, _vp, _WP, _vp,
                            _vp, _vp, _vp, _vp, C.c_size_t, C.POINTER(_vp), _i32, _vp)
_fused_forward_noalloc = _sig("moe_fused_forward_noalloc", _i32, _DP, _vp, _vp, _vp, _vp, _WP,
                              _vp, _vp, _vp, _vp, _vp)
_group_tokens = _sig("moe_group_tokens", _i32, _vp, _i32, _i32, _i32, _i32, _vp)
_k_tiers = _sig("moe_k_tiers", _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp)

N_STAGE_EVENTS = 8
STAGES = ("route", "topk", "permute", "gate_up", "requant", "down", "combine")

ABI_VERSION = int(_abi_version())
STATIC_WORKSPACE_BYTES = 128 << 20  # MOE_STATIC_WORKSPACE_BYTES


class MoEError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        detail = _last_error().decode()
        super().__init__(f"{_status_str(status).decode()} ({status}): {detail}")


def _check(status: int):
    if status != 0:
        raise MoEError(status)


def _ptr(t: Optional[torch.Tensor], dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("fp8_moe_layer_amd works on device tensors only")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _on(stream):
    """Context in which new tensors are allocated for `stream` (the caching
    allocator then never hands their memory to another stream while work on
    this one may still use it)."""
    import contextlib
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


# --------------------------------------------------------------------------- steps

def quantize_rows(x: torch.Tensor, q: Optional[torch.Tensor] = None, scale=None, stream=None):
    """Per-row e4m3 quantisation: (codes uint8 like x, fp32 scale per row)."""
    cols = x.shape[-1]
    rows = x.numel() // cols
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device) if scale is None else scale
    _check(_quantize_rows(_ptr(x, torch.float32), rows, cols, _ptr(q, torch.uint8),
                          _ptr(scale, torch.float32), _stream(stream)))
    return q, scale


def packed_weight_bytes(rows: int, cols: int) -> int:
    """Bytes of a [rows][cols] code matrix in tile order (0 for bad shapes)."""
    return int(_packed_weight_bytes(rows, cols))


def packed_shape(rows: int, cols: int):
    """Tensor shape used for one tile-order matrix: [rows/16, ceil(cols/128), 2048]."""
    return (rows // 16, (cols + 127) // 128, 2048)


def pack_weights(codes: torch.Tensor, packed: Optional[torch.Tensor] = None, stream=None):
    """Row-major e4m3 codes [rows][cols] -> tile order (the layout the
    expert GEMMs read; see moe_weights in include/fp8moe.h)."""
    rows, cols = codes.shape
    if packed is None:
        packed = torch.empty(packed_shape(rows, cols), dtype=torch.uint8, device=codes.device)
    need = packed_weight_bytes(rows, cols)  # 0: a bad shape, reported by the library
    if need and packed.numel() != need:
        raise ValueError(f"packed holds {packed.numel()} bytes, {need} needed")
    _check(_pack_weights(_ptr(codes, torch.uint8), rows, cols, _ptr(packed, torch.uint8),
                         _stream(stream)))
    return packed


def router_logits(x, w_router, bias=None, stream=None):
    T, d = x.shape
    E = w_router.shape[0]
    out = torch.empty((T, E), dtype=torch.float32, device=x.device)
    _check(_router_logits(_ptr(x, torch.float32), _ptr(w_router, torch.float32),
                          _ptr(bias, torch.float32), T, d, E, _ptr(out), _stream(stream)))
    return out


def route_topk(logits, k_max: int, k_per_token=None, stream=None):
    T, E = logits.shape
    ids = torch.empty((T, k_max), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, k_max), dtype=torch.float32, device=logits.device)
    _check(_route_topk(_ptr(logits, torch.float32), T, E, k_max, _ptr(k_per_token, torch.int32),
                       _ptr(ids), _ptr(w), _stream(stream)))
    return ids, w


def group_tokens(topk_ids, E: int, batch: int):
    """Order a token pool into decode batches of `batch` tokens that activate
    few distinct experts (moe_group_tokens; host computation).  topk_ids:
    [n, k] int32 routing (numpy or a torch tensor, copied to the host).
    Returns the order, an int32 numpy permutation of range(n)."""
    import numpy as np
    if isinstance(topk_ids, torch.Tensor):
        topk_ids = topk_ids.detach().cpu().numpy()
    ids = np.ascontiguousarray(topk_ids, dtype=np.int32)
    n, k = ids.shape
    order = np.empty(n, dtype=np.int32)
    _check(_group_tokens(ids.ctypes.data if n else None, n, k, E, batch,
                         order.ctypes.data if n else None))
    return order


def k_tiers(k_per_token, batch: int, overhead: int):
    """Plan quality-tier batches of a pool by routing budget (moe_k_tiers;
    host computation).  k_per_token: [n] int32 budgets (numpy or a torch
    tensor, copied to the host).  Returns (order, batch_start, batch_k):
    batch b is order[batch_start[b]:batch_start[b+1]], run at k batch_k[b]."""
    import numpy as np
    if isinstance(k_per_token, torch.Tensor):
        k_per_token = k_per_token.detach().cpu().numpy()
    kpt = np.ascontiguousarray(k_per_token, dtype=np.int32).reshape(-1)
    n = kpt.size
    order = np.empty(n, dtype=np.int32)
    start = np.empty(n + 1, dtype=np.int32)
    bk = np.empty(max(n, 1), dtype=np.int32)
    nb = np.zeros(1, dtype=np.int32)
    _check(_k_tiers(kpt.ctypes.data if n else None, n, batch, overhead,
                    order.ctypes.data if n else None, start.ctypes.data,
                    bk.ctypes.data if n else None, nb.ctypes.data))
    m = int(nb[0])
    return order, start[:m + 1].copy(), bk[:m].copy()


def capacity(T: int, E: int, k_max: int, block_m: int) -> int:
    return int(_capacity(T, E, k_max, block_m))


def permute_workspace_bytes(T: int, E: int, k_max: int) -> int:
    return int(_permute_ws_bytes(T, E, k_max))


def permute(topk_ids, E: int, block_m: int, cap: Optional[int] = None, stream=None,
            workspace: bool = False) -> dict:
    """moe_permute, or with workspace=True moe_permute_ws on a workspace
    allocated here (the two-launch form for large batches)."""
    T, K = topk_ids.shape
    cap = capacity(T, E, K, block_m) if cap is None else cap
    dev = topk_ids.device
    z = lambda n: torch.empty(n, dtype=torch.int32, device=dev)
    out = dict(sorted_pairs=z(cap), expert_offsets=z(E + 1), block_expert=z((cap + block_m - 1) // block_m),
               inv_pairs=z(T * K), n_blocks=z(1))
    args = (_ptr(topk_ids, torch.int32), T, E, K, block_m, cap, _ptr(out["sorted_pairs"]),
            _ptr(out["expert_offsets"]), _ptr(out["block_expert"]), _ptr(out["inv_pairs"]),
            _ptr(out["n_blocks"]))
    if workspace:
        n = permute_workspace_bytes(T, E, K)
        with _on(stream):
            ws = torch.empty(max(n, 16), dtype=torch.uint8, device=dev)
        _check(_permute_ws(*args, _ptr(ws), n, _stream(stream)))
        out["workspace"] = ws  # kept alive with the outputs until the caller syncs
    else:
        _check(_permute(*args, _stream(stream)))
    out["capacity"] = cap
    return out


# --------------------------------------------------------------------------- weights

@dataclass
class DeviceWeights:
    """e4m3 expert weights with fp32 per-output-channel scales.  The codes are
    kept in tile order (pack_weights): one [f/16, ceil(d/128), 2048] block per
    expert for gate and up, [d/16, ceil(f/128), 2048] for down."""
    w_gate: torch.Tensor  # [E, f/16, ceil(d/128), 2048]
    w_up: torch.Tensor
    s_gate: torch.Tensor  # [E, f]
    s_up: torch.Tensor
    w_down: torch.Tensor  # [E, d/16, ceil(f/128), 2048]
    s_down: torch.Tensor  # [E, d]
    ws_gate: Optional[torch.Tensor] = None
    ws_up: Optional[torch.Tensor] = None
    ss_gate: Optional[torch.Tensor] = None
    ss_up: Optional[torch.Tensor] = None
    ws_down: Optional[torch.Tensor] = None
    ss_down: Optional[torch.Tensor] = None

    @property
    def E(self) -> int:
        return int(self.w_gate.shape[0])

    @property
    def f(self) -> int:
        return int(self.s_gate.shape[1])

    @property
    def d(self) -> int:
        return int(self.s_down.shape[1])

    @property
    def n_shared(self) -> int:
        return 0 if self.ws_gate is None else int(self.ws_gate.shape[0])

    def struct(self) -> _Weights:
        p = lambda t: _ptr(t)
        return _Weights(p(self.w_gate), p(self.w_up), p(self.s_gate), p(self.s_up), p(self.w_down),
                        p(self.s_down), p(self.ws_gate), p(self.ws_up), p(self.ws_down),
                        p(self.ss_gate), p(self.ss_up), p(self.ss_down))

    @staticmethod
    def empty(E: int, d: int, f: int, n_shared: int = 0, device="cuda") -> "DeviceWeights":
        u8 = lambda n, r, c: torch.empty((n,) + packed_shape(r, c), dtype=torch.uint8, device=device)
        f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=device)
        w = DeviceWeights(u8(E, f, d), u8(E, f, d), f32(E, f), f32(E, f), u8(E, d, f), f32(E, d))
        if n_shared:
            S = n_shared
            w.ws_gate, w.ws_up, w.ws_down = u8(S, f, d), u8(S, f, d), u8(S, d, f)
            w.ss_gate, w.ss_up, w.ss_down = f32(S, f), f32(S, f), f32(S, d)
        return w

    def set_expert(self, which: str, e: int, w32: torch.Tensor, shared: bool = False):
        """Quantise one fp32 expert matrix [rows][cols] per output channel and
        store it in tile order in slot e."""
        pre = "ws_" if shared else "w_"
        spre = "ss_" if shared else "s_"
        codes, _ = quantize_rows(w32.contiguous(), scale=getattr(self, spre + which)[e])
        pack_weights(codes, getattr(self, pre + which)[e])


# --------------------------------------------------------------------------- expert stages

def dims(T, d, f, E, k_max, n_shared=0, block_m=16, no_requant=False, persistent=False) -> Dims:
    flags = (MOE_F_NO_REQUANT if no_requant else 0) | (MOE_F_PERSISTENT if persistent else 0)
    return Dims(T, d, f, E, k_max, n_shared, block_m, flags)


def expert_gate_up(dm: Dims, perm: dict, xq, sx, w: DeviceWeights, stream=None):
    rows = perm["capacity"] + dm.n_shared * dm.T
    h = torch.zeros((rows, dm.f), dtype=torch.float32, device=xq.device)
    ws = w.struct()
    _check(_gate_up(C.byref(dm), perm["capacity"], _ptr(xq, torch.uint8), _ptr(sx, torch.float32),
                    _ptr(perm["sorted_pairs"]), _ptr(perm["expert_offsets"]), C.byref(ws), _ptr(h),
                    _stream(stream)))
    return h


def expert_down(dm: Dims, perm: dict, w: DeviceWeights, hq=None, sh=None, h=None, stream=None):
    rows = perm["capacity"] + dm.n_shared * dm.T
    dev = (hq if hq is not None else h).device
    y = torch.zeros((rows, dm.d), dtype=torch.float32, device=dev)
    ws = w.struct()
    _check(_down(C.byref(dm), perm["capacity"], _ptr(hq, torch.uint8), _ptr(sh, torch.float32),
                 _ptr(h, torch.float32), _ptr(perm["sorted_pairs"]), _ptr(perm["expert_offsets"]),
                 C.byref(ws), _ptr(y), _stream(stream)))
    return y


def combine(dm: Dims, perm: dict, y, topk_ids, topk_w, stream=None):
    out = torch.empty((dm.T, dm.d), dtype=torch.float32, device=y.device)
    _check(_combine(C.byref(dm), perm["capacity"], _ptr(y, torch.float32), _ptr(topk_ids, torch.int32),
                    _ptr(topk_w, torch.float32), _ptr(perm["inv_pairs"]), _ptr(out), _stream(stream)))
    return out


# --------------------------------------------------------------------------- whole layer

def workspace_bytes(dm: Dims) -> int:
    return int(_workspace_bytes(C.byref(dm)))


class DebugLibrary:
    """The device-checked build of the same sources (libfp8moe_debug.so,
    compiled with FP8MOE_DEBUG): kernels check the layer's preconditions
    (k_per_token in [1, k_max], finite logits and activations, top-k ids in
    [-1, E)) and the permutation's index invariants; every call that enqueues
    work waits for it and returns MOE_ERR_DEVICE_CHECK (7) naming the failed
    checks.  It synchronises, so it is for testing, not for timing or graph
    capture.  Calls return (status, error text) instead of raising."""

    def __init__(self):
        if not DEBUG_LIB_PATH.exists():
            raise ImportError(f"{DEBUG_LIB_PATH} is not built (fp8_moe_layer_amd/build.py --debug)")
        lib = C.CDLL(str(DEBUG_LIB_PATH))

        def sig(name, restype, *argtypes):
            fn = getattr(lib, name)
            fn.restype = restype
            fn.argtypes = list(argtypes)
            return fn

        self._fwd = sig("moe_fused_forward", _i32, _DP, _vp, _vp, _vp, _vp, _WP, _vp, _vp, _vp,
                        _vp, _vp, C.c_size_t, _vp)
        self._topk = sig("moe_route_topk", _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp)
        self._permute = sig("moe_permute", _i32, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                            _vp, _vp, _vp, _vp)
        self.workspace_bytes = sig("moe_workspace_bytes", C.c_size_t, _DP)
        self.status_str = sig("moe_status_str", C.c_char_p, _i32)
        self._last_error = sig("moe_last_error", C.c_char_p)
        self.checks = int(sig("moe_debug_checks", _i32)())

    def _result(self, rc: int):
        return int(rc), (self._last_error() or b"").decode()

    def forward(self, layer: "MoELayer", x: torch.Tensor, k_per_token=None, logits_override=None,
                out=None, topk_ids=None, stream=None):
        """layer's forward through the debug build: (status, text, out)."""
        T = x.shape[0]
        dm = layer.dims(T)
        if out is None:
            out = torch.empty((T, layer.w.d), dtype=torch.float32, device=x.device)
        n = int(self.workspace_bytes(C.byref(dm)))
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=x.device)
        rc = self._fwd(C.byref(dm), _ptr(x, torch.float32), _ptr(layer.w_router, torch.float32),
                       _ptr(layer.router_bias, torch.float32), _ptr(k_per_token, torch.int32),
                       C.byref(layer._wstruct), _ptr(logits_override, torch.float32), _ptr(out),
                       _ptr(topk_ids, torch.int32), None, _ptr(ws), n, _stream(stream))
        return (*self._result(rc), out)

    def route_topk(self, logits: torch.Tensor, k_max: int, k_per_token=None, stream=None):
        """(status, text, ids, w) of moe_route_topk through the debug build."""
        T, E = logits.shape
        ids = torch.empty((T, k_max), dtype=torch.int32, device=logits.device)
        w = torch.empty((T, k_max), dtype=torch.float32, device=logits.device)
        rc = self._topk(_ptr(logits, torch.float32), T, E, k_max, _ptr(k_per_token, torch.int32),
                        _ptr(ids), _ptr(w), _stream(stream))
        return (*self._result(rc), ids, w)

    def permute(self, topk_ids: torch.Tensor, E: int, block_m: int = 16, stream=None):
        """(status, text) of moe_permute through the debug build."""
        T, k = topk_ids.shape
        cap = capacity(T, E, k, block_m)
        dv = topk_ids.device
        i32 = dict(dtype=torch.int32, device=dv)
        sp, off = torch.empty(cap, **i32), torch.empty(E + 1, **i32)
        be = torch.empty((cap + block_m - 1) // block_m, **i32)
        inv, nb = torch.empty(T * k, **i32), torch.empty(1, **i32)
        rc = self._permute(_ptr(topk_ids, torch.int32), T, E, k, block_m, cap, _ptr(sp), _ptr(off),
                           _ptr(be), _ptr(inv), _ptr(nb), _stream(stream))
        return self._result(rc)


class MoELayer:
    """One W8A8 FP8 MoE layer resident on the device.

    forward(x) runs the whole layer (quantise, router, top-k, permutation,
    gate/up + SiLU*up, requantisation, down projection, combine) in the
    library's kernels on the current stream -- six launches at decode sizes,
    eight to ten at prefill sizes, or (persistent=True) one cooperative
    launch after a one-wave reset.  The workspace is allocated once per
    token count and reused.
    """

    def __init__(self, weights: DeviceWeights, w_router: Optional[torch.Tensor], k_max: int,
                 router_bias: Optional[torch.Tensor] = None, block_m: int = 16,
                 no_requant: bool = False, persistent: bool = False):
        self.w = weights
        self.w_router = w_router
        self.router_bias = router_bias
        self.k_max = k_max
        self.block_m = block_m
        self.no_requant = no_requant
        self.persistent = persistent
        self._ws = {}
        self._wstruct = weights.struct()

    def dims(self, T: int) -> Dims:
        return dims(T, self.w.d, self.w.f, self.w.E, self.k_max, self.w.n_shared, self.block_m,
                    self.no_requant, self.persistent)

    def workspace(self, T: int, device, stream=None) -> torch.Tensor:
        """The workspace for T tokens, allocated on `stream` (the stream the
        layer's kernels will use) and kept until T changes."""
        key = (T, None if stream is None else stream.cuda_stream)
        ws = self._ws.get(key)
        if ws is None:
            n = workspace_bytes(self.dims(T))
            if n == 0:
                raise MoEError(int(2))
            with _on(stream):
                ws = torch.empty(n, dtype=torch.uint8, device=device)
            self._ws = {key: ws}
        return ws

    def forward(self, x: torch.Tensor, k_per_token=None, logits_override=None, out=None,
                topk_ids=None, topk_w=None, stream=None, stage_events=None) -> torch.Tensor:
        """stream: a torch.cuda.Stream (default: the current one); stage_events:
        MOE_N_STAGE_EVENTS hipEvent_t handles recorded around the stages
        (instrumentation), or None."""
        T = x.shape[0]
        dm = self.dims(T)
        if out is None:
            with _on(stream):
                out = torch.empty((T, self.w.d), dtype=torch.float32, device=x.device)
        ws = self.workspace(T, x.device, stream)
        ev = None if stage_events is None else (_vp * len(stage_events))(*stage_events)
        _check(_fused_forward_timed(
            C.byref(dm), _ptr(x, torch.float32), _ptr(self.w_router, torch.float32),
            _ptr(self.router_bias, torch.float32), _ptr(k_per_token, torch.int32),
            C.byref(self._wstruct), _ptr(logits_override, torch.float32), _ptr(out),
            _ptr(topk_ids, torch.int32), _ptr(topk_w, torch.float32), _ptr(ws), ws.numel(), ev,
            0 if ev is None else len(stage_events), _stream(stream)))
        return out

    def status(self) -> int:
        """The persistent launch's status word (workspace offset 0): 0 = ok,
        1 = a grid barrier timed out.  Synchronises; meaningful only after a
        forward with persistent=True."""
        if not self.persistent or not self._ws:
            return 0
        ws = next(iter(self._ws.values()))
        return int(ws[:4].view(torch.int32).item())

    def persistent_stamps(self):
        """Microseconds from the persistent launch's start to each of its
        recorded phase boundaries (workgroup 0's clock: after each grid
        barrier, then the end).  Synchronises; after a persistent forward."""
        if not self.persistent or not self._ws:
            return []
        ws = next(iter(self._ws.values()))
        off = 34 * 65536  # the stamps slot of the barrier state
        st = ws[off:off + 80].view(torch.int64).cpu().tolist()
        t0 = st[0]
        return [round((v - t0) / 100.0, 2) for v in st[1:] if v >= t0 and v - t0 < 10**9]

    def forward_noalloc(self, x: torch.Tensor, out: torch.Tensor, k_per_token=None,
                        logits_override=None, topk_ids=None, topk_w=None, stream=None):
        """The same forward through moe_fused_forward_noalloc: the library's
        own static device workspace, no allocation by the library or here
        (out is the caller's).  Calls overlapping on one GPU race."""
        T = x.shape[0]
        dm = self.dims(T)
        _check(_fused_forward_noalloc(
            C.byref(dm), _ptr(x, torch.float32), _ptr(self.w_router, torch.float32),
            _ptr(self.router_bias, torch.float32), _ptr(k_per_token, torch.int32),
            C.byref(self._wstruct), _ptr(logits_override, torch.float32), _ptr(out, torch.float32),
            _ptr(topk_ids, torch.int32), _ptr(topk_w, torch.float32), _stream(stream)))
        return out

    __call__ = forward
