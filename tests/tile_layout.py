"""The tile order of expert weight codes, written out from its definition in
include/fp8moe.h (moe_weights), for the tests: W[r][c] of an R x C matrix
(R % 16 == 0, C % 64 == 0) lives in 2048-byte tile (r // 16) * CT + c // 128,
CT = ceil(C / 128), at byte l * 16 + c % 16 (c % 128 < 64) or
1024 + l * 16 + c % 16 (c % 128 >= 64), with l = r % 16 + 16 * ((c % 64) // 16);
bytes for c >= C are zero."""
import numpy as np


def tile_offset(r: int, c: int, C: int) -> int:
    CT = (C + 127) // 128
    l = r % 16 + 16 * ((c % 64) // 16)
    inner = l * 16 + c % 16 + (1024 if c % 128 >= 64 else 0)
    return ((r // 16) * CT + c // 128) * 2048 + inner


def pack(codes: np.ndarray) -> np.ndarray:
    """[..., R, C] row-major codes -> [..., R/16, CT, 2048] tile order."""
    *lead, R, C = codes.shape
    CT = (C + 127) // 128
    padded = np.zeros((*lead, R, CT * 128), np.uint8)
    padded[..., :C] = codes
    # r = 16*rt + ln ; c = 128*ct + 64*half + 16*kg + j
    v = padded.reshape(*lead, R // 16, 16, CT, 2, 4, 16)      # rt, ln, ct, half, kg, j
    n = len(lead)
    perm = list(range(n)) + [n + 0, n + 2, n + 3, n + 4, n + 1, n + 5]  # rt, ct, half, kg, ln, j
    return np.ascontiguousarray(v.transpose(perm)).reshape(*lead, R // 16, CT, 2048)


def unpack(packed: np.ndarray, R: int, C: int) -> np.ndarray:
    """Inverse of pack: [..., R/16, CT, 2048] -> [..., R, C]."""
    *lead, RT, CT, _ = packed.shape
    assert RT * 16 == R and CT == (C + 127) // 128
    v = packed.reshape(*lead, RT, CT, 2, 4, 16, 16)           # rt, ct, half, kg, ln, j
    n = len(lead)
    perm = list(range(n)) + [n + 0, n + 4, n + 1, n + 2, n + 3, n + 5]  # rt, ln, ct, half, kg, j
    full = np.ascontiguousarray(v.transpose(perm)).reshape(*lead, R, CT * 128)
    return full[..., :C]
