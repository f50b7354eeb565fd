"""C-ABI checks that need no GPU: the HIP library loads, exports every entry
point declared in include/fp8moe.h, and rejects bad arguments on the host
before anything is enqueued (each call below fails validation, so no kernel
is ever launched)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8moe.h")

fp8 = pytest.importorskip("fp8_moe_layer_amd", reason="libfp8moe.so not built")

OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_DEVICE_CHECK = range(8)
FAKE = 0x10000  # an aligned non-null address; never dereferenced (validation fails first)


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.mark.parametrize("debug", [False, True])
def test_every_declared_symbol_is_exported(debug):
    names = _declared()
    assert len(names) >= 13
    path = fp8.DEBUG_LIB_PATH if debug else fp8.LIB_PATH
    if debug and not path.exists():
        pytest.skip("libfp8moe_debug.so not built")
    lib = C.CDLL(str(path))
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    # the release library reports no device checks, the debug build does
    assert lib.moe_debug_checks() == (1 if debug else 0)


def test_debug_library_rejects_on_the_host_like_the_release_one():
    if not fp8.DEBUG_LIB_PATH.exists():
        pytest.skip("libfp8moe_debug.so not built")
    dbg = fp8.DebugLibrary()
    assert dbg.checks == 1
    bad = fp8.dims(0, 256, 512, 8, 2, 0, 16)
    assert dbg.workspace_bytes(C.byref(bad)) == 0
    assert dbg.status_str(ERR_DEVICE_CHECK) == b"device check failed (debug build)"


def test_abi_version_and_status_strings():
    assert fp8.ABI_VERSION == 6
    assert fp8._status_str(ERR_DEVICE_CHECK) == b"device check failed (debug build)"
    assert fp8._status_str(0) == b"ok"
    assert fp8._status_str(ERR_WORKSPACE) == b"workspace too small"
    assert fp8._status_str(99) == b"unknown status"


def test_capacity_formula():
    assert fp8.capacity(16, 8, 2, 16) == 16 * 2 + 8 * 15
    assert fp8.capacity(1024, 512, 32, 1) == 1024 * 32


def _dims(**kw):
    base = dict(T=16, d=256, f=512, E=8, k_max=2, n_shared=0, block_m=16, no_requant=False)
    base.update(kw)
    return fp8.dims(**base)


def test_workspace_bytes():
    small = fp8.workspace_bytes(_dims(T=16))
    big = fp8.workspace_bytes(_dims(T=1024))
    assert 0 < small < big
    assert fp8.workspace_bytes(_dims(T=0)) == 0           # invalid dims -> 0
    assert fp8.workspace_bytes(_dims(block_m=7)) == 0
    # Mixtral-shaped decode layer fits comfortably
    mix = fp8.workspace_bytes(_dims(T=256, d=4096, f=14336, E=8, k_max=2))
    assert mix < 512 << 20


@pytest.mark.parametrize("kw,code", [
    (dict(T=0), ERR_SHAPE),
    (dict(d=100), ERR_SHAPE),
    (dict(f=96), ERR_SHAPE),
    (dict(E=0), ERR_SHAPE),
    (dict(E=513, k_max=2), ERR_SHAPE),
    (dict(k_max=9), ERR_SHAPE),
    (dict(E=64, k_max=33), ERR_SHAPE),
    (dict(block_m=24), ERR_SHAPE),
    (dict(n_shared=-1), ERR_SHAPE),
])
def test_fused_forward_rejects_bad_dims(kw, code):
    dm = _dims(**kw)
    w = fp8._Weights(*([FAKE] * 12))
    rc = fp8._fused_forward(C.byref(dm), FAKE, FAKE, None, None, C.byref(w), None, FAKE, None, None,
                            FAKE, 1 << 40, None)
    assert rc == code, fp8._last_error()
    assert fp8._last_error()


def test_fused_forward_rejects_null_and_alignment_and_workspace():
    dm = _dims()
    w = fp8._Weights(*([FAKE] * 12))
    call = lambda **kw: fp8._fused_forward(
        C.byref(kw.get("dims", dm)), kw.get("x", FAKE), kw.get("wr", FAKE), None, None,
        C.byref(kw.get("w", w)), kw.get("lo", None), kw.get("out", FAKE), None, None,
        kw.get("ws", FAKE), kw.get("wsb", 1 << 40), None)
    assert fp8._fused_forward(None, FAKE, FAKE, None, None, C.byref(w), None, FAKE, None, None,
                              FAKE, 1 << 40, None) == ERR_NULL
    assert call(x=None) == ERR_NULL
    assert call(wr=None) == ERR_NULL                       # no router and no override
    assert call(x=FAKE + 4) == ERR_ALIGN
    assert call(ws=FAKE + 16) == ERR_ALIGN
    assert call(ws=None) == ERR_WORKSPACE
    assert call(wsb=fp8.workspace_bytes(dm) - 1) == ERR_WORKSPACE
    w2 = fp8._Weights(*([FAKE] * 12))
    w2.w_down = None
    assert call(w=w2) == ERR_NULL
    w3 = fp8._Weights(*([FAKE] * 12))
    w3.w_gate = FAKE + 8
    assert call(w=w3) == ERR_ALIGN
    sh = _dims(n_shared=2)
    w4 = fp8._Weights(*([FAKE] * 6 + [None] * 6))
    assert call(dims=sh, w=w4) == ERR_NULL
    bad_flags = _dims()
    bad_flags.flags = 1 << 5
    assert call(dims=bad_flags) == ERR_UNSUPPORTED
    # the fused combine is not built: refused, on every call that takes dims
    fc = _dims()
    fc.flags = fp8.MOE_F_FUSED_COMBINE
    assert call(dims=fc) == ERR_UNSUPPORTED
    assert b"MOE_F_FUSED_COMBINE" in fp8._last_error()
    assert fp8.workspace_bytes(fc) == 0
    cap = fp8.capacity(16, 8, 2, 16)
    assert fp8._gate_up(C.byref(fc), cap, FAKE, FAKE, FAKE, FAKE, C.byref(w), FAKE, None) == ERR_UNSUPPORTED
    assert fp8._combine(C.byref(fc), cap, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ERR_UNSUPPORTED
    # the single-launch flag: its workspace adds the grid-barrier state (2.2 MB,
    # the status word first); everything else is validated as for the staged path
    for extra in (0, fp8.MOE_F_NO_REQUANT):
        pers = _dims()
        pers.flags = fp8.MOE_F_PERSISTENT | extra
        stg = _dims()
        stg.flags = extra
        assert fp8.workspace_bytes(pers) >= fp8.workspace_bytes(stg) + 34 * 65536
        assert call(dims=pers, x=None) == ERR_NULL
        assert call(dims=pers, wsb=fp8.workspace_bytes(pers) - 1) == ERR_WORKSPACE


def test_timed_forward_checks_its_events_and_keeps_no_pointer():
    """moe_fused_forward_timed takes the stage events as an argument of the
    call (the library keeps no caller pointer between calls) and refuses a
    short event array before anything is enqueued."""
    dm = _dims()
    w = fp8._Weights(*([FAKE] * 12))
    ev = (C.c_void_p * fp8.N_STAGE_EVENTS)(*([FAKE] * fp8.N_STAGE_EVENTS))
    timed = lambda events, n, wsb=1 << 40: fp8._fused_forward_timed(
        C.byref(dm), FAKE, FAKE, None, None, C.byref(w), None, FAKE, None, None, FAKE, wsb,
        events, n, None)
    assert timed(ev, fp8.N_STAGE_EVENTS - 1) == ERR_SHAPE
    assert b"stage events" in fp8._last_error()
    # with no events it validates exactly like moe_fused_forward
    assert timed(None, 0, wsb=16) == ERR_WORKSPACE
    assert timed(ev, fp8.N_STAGE_EVENTS, wsb=16) == ERR_WORKSPACE
    assert not hasattr(C.CDLL(str(fp8.LIB_PATH)), "moe_debug_stage_events")


def test_noalloc_forward_refuses_before_touching_the_device():
    """moe_fused_forward_noalloc validates like moe_fused_forward and refuses
    dims whose workspace exceeds the static array, all before any device
    call (so these run without a GPU)."""
    w = fp8._Weights(*([FAKE] * 12))
    na = lambda dm, x=FAKE: fp8._fused_forward_noalloc(C.byref(dm), x, FAKE, None, None, C.byref(w),
                                                       None, FAKE, None, None, None)
    assert na(_dims(T=0)) == ERR_SHAPE
    assert na(_dims(), x=None) == ERR_NULL
    big = _dims(T=4096, d=2048, f=768, E=128, k_max=8)
    assert fp8.workspace_bytes(big) > fp8.STATIC_WORKSPACE_BYTES
    assert na(big) == ERR_WORKSPACE
    assert b"static scratch" in fp8._last_error()


def test_packed_weight_bytes_and_pack_validation():
    assert fp8.packed_weight_bytes(16, 64) == 16 * 128          # tail padded to a full tile
    assert fp8.packed_weight_bytes(32, 256) == 32 * 256
    assert fp8.packed_weight_bytes(4096, 14336) == 4096 * 14336
    for r, c in ((0, 64), (8, 64), (16, 32), (16, 0), (-16, 64)):
        assert fp8.packed_weight_bytes(r, c) == 0
    assert fp8._pack_weights(None, 16, 64, FAKE, None) == ERR_NULL
    assert fp8._pack_weights(FAKE, 24, 64, FAKE + (1 << 30), None) == ERR_SHAPE
    assert fp8._pack_weights(FAKE, 16, 16384 + 64, FAKE + (1 << 30), None) == ERR_SHAPE
    assert fp8._pack_weights(FAKE + 4, 16, 64, FAKE + (1 << 30), None) == ERR_ALIGN
    assert fp8._pack_weights(FAKE, 16, 128, FAKE + 1024, None) == ERR_SHAPE  # overlap


def test_step_entry_points_reject_bad_arguments():
    assert fp8._quantize_rows(None, 4, 8, FAKE, FAKE, None) == ERR_NULL
    assert fp8._quantize_rows(FAKE, 4, 6, FAKE, FAKE, None) == ERR_SHAPE
    assert fp8._quantize_rows(FAKE + 4, 4, 8, FAKE, FAKE, None) == ERR_ALIGN
    assert fp8._router_logits(FAKE, FAKE, None, 4, 100, 8, FAKE, None) == ERR_SHAPE
    assert fp8._router_logits(FAKE, None, None, 4, 128, 8, FAKE, None) == ERR_NULL
    assert fp8._route_topk(FAKE, 4, 8, 9, None, FAKE, FAKE, None) == ERR_SHAPE
    assert fp8._route_topk(FAKE, 4, 600, 2, None, FAKE, FAKE, None) == ERR_SHAPE
    assert fp8._route_topk(FAKE, 4, 64, 33, None, FAKE, FAKE, None) == ERR_SHAPE
    assert fp8._permute(FAKE, 4, 8, 2, 16, 10, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert fp8._permute(FAKE, 4, 8, 2, 3, 1000, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert fp8._permute(FAKE, 4, 8, 2, 16, 1000, None, FAKE, FAKE, FAKE, FAKE, None) == ERR_NULL
    # the workspace form: 4096 pairs or more need slice counts (4 slices x E ints)
    assert fp8.permute_workspace_bytes(16, 8, 2) == 0
    assert fp8.permute_workspace_bytes(2048, 64, 2) == 4 * 64 * 4
    assert fp8.permute_workspace_bytes(8192, 64, 6) == 48 * 64 * 4
    cap = fp8.capacity(2048, 64, 2, 16)
    assert fp8._permute_ws(FAKE, 2048, 64, 2, 16, cap, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0,
                           None) == ERR_WORKSPACE
    assert fp8._permute_ws(FAKE, 2048, 64, 2, 16, cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 100,
                           None) == ERR_WORKSPACE
    assert fp8._permute_ws(FAKE, 2048, 64, 2, 16, cap, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, 1024,
                           None) == ERR_ALIGN
    assert fp8._permute_ws(FAKE, 2048, 64, 2, 16, cap - 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1024,
                           None) == ERR_SHAPE
    dm = _dims()
    w = fp8._Weights(*([FAKE] * 12))
    cap = fp8.capacity(16, 8, 2, 16)
    assert fp8._gate_up(C.byref(dm), cap - 1, FAKE, FAKE, FAKE, FAKE, C.byref(w), FAKE, None) == ERR_SHAPE
    assert fp8._gate_up(C.byref(dm), cap, None, FAKE, FAKE, FAKE, C.byref(w), FAKE, None) == ERR_NULL
    assert fp8._down(C.byref(dm), cap, None, FAKE, None, FAKE, FAKE, C.byref(w), FAKE, None) == ERR_NULL
    nr = _dims(no_requant=True)
    assert fp8._down(C.byref(nr), cap, FAKE, FAKE, None, FAKE, FAKE, C.byref(w), FAKE, None) == ERR_NULL
    assert fp8._combine(C.byref(dm), cap, FAKE, FAKE, FAKE, None, FAKE, None) == ERR_NULL
    assert fp8._combine(C.byref(dm), 3, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ERR_SHAPE
    assert b"capacity" in fp8._last_error()
