"""A model of the workgroup and grid barriers the GEMM tiles and the
persistent kernel execute, checked on the CPU: every wave of a workgroup
must execute the same number of s_barrier instructions per tile (the loader
wave and the compute waves of the row-pass tile take different code paths),
and every workgroup of the persistent grid the same sequence of grid
barriers, or the launch would deadlock.  The counts are those of the loops in
csrc/expert_dev.hpp (wsgemm_tile, pf_tile) and csrc/kernels_persistent.hip,
restated here."""
import itertools

import pytest


def chunk_geometry(msub):
    """K steps per LDS chunk, weight prefetch depth (the Chunk<MSUB> constants)."""
    ksc = 1 if msub >= 8 else 8 // msub
    pf = 4 if msub <= 2 else 2
    return ksc, pf


def rowpass_barriers(msub, rows, k_bytes):
    """(loader, compute) s_barrier counts of one wsgemm_tile call."""
    ksc, pf = chunk_geometry(msub)
    nks = (k_bytes + 127) // 128
    nks_pf = (nks + pf - 1) // pf * pf
    nchunks = (nks_pf + ksc - 1) // ksc
    passes = (rows + 16 * msub - 1) // (16 * msub)
    nbuf = 4
    # loader: one wait-barrier for chunk 0, then one per chunk of the loop
    loader = 0
    for _ in range(passes):
        pre = min(nbuf - 1, nchunks)
        loader += 1
        for c in range(nchunks):
            loader += 1
    # compute: one after the first weight loads, one at the end of each chunk
    compute = 0
    for _ in range(passes):
        compute += 1
        for ks in range(nks_pf):
            if (ks + 1) % ksc == 0 or ks + 1 == nks_pf:
                compute += 1
    return loader, compute


@pytest.mark.parametrize("msub", [1, 2, 4, 8, 16])
def test_rowpass_tile_waves_meet_at_every_barrier(msub):
    for rows, k in itertools.product((1, 15, 16, 17, 127, 128, 129, 256, 300, 1024),
                                     (64, 128, 192, 256, 768, 1408, 2048, 4096, 14336)):
        loader, compute = rowpass_barriers(msub, rows, k)
        assert loader == compute, (msub, rows, k, loader, compute)


def prefill_barriers(rows, k_bytes):
    """s_barrier count of one pf_tile call (every wave runs the same loop)."""
    pf = 2
    nks = (k_bytes + 127) // 128
    nch = (nks + pf - 1) // pf * pf
    passes = (rows + 255) // 256
    return passes * (1 + nch)


def test_prefill_tile_is_symmetric():
    # one code path for all eight waves: the count depends only on the item
    for rows, k in itertools.product((1, 255, 256, 257, 3072), (192, 768, 1408, 2048)):
        assert prefill_barriers(rows, k) > 0


def persistent_grid_barriers(T, E, logits_override, requant):
    """Grid barriers of the persistent kernel for one launch (the same for
    every workgroup: no phase is skipped by one workgroup only)."""
    dot = T * E <= 65536
    topk_fused = (not logits_override) and (not dot) and E <= 128
    n = 1                      # after routing
    n += 0 if topk_fused else 1  # after top-k
    n += 1                     # after the permutation (workgroup 0 works, all wait)
    n += 1                     # after gate/up
    n += 1 if requant else 0   # after the requantisation
    n += 1                     # after the down projection
    return n


@pytest.mark.parametrize("T,E", [(1, 8), (256, 8), (64, 128), (4096, 128), (8192, 64),
                                 (1024, 512), (40, 8)])
def test_persistent_barrier_sequence(T, E):
    for lo, rq in itertools.product((False, True), (False, True)):
        n = persistent_grid_barriers(T, E, lo, rq)
        # the barrier generations 1..n are passed in order by every workgroup
        assert 4 <= n <= 6
