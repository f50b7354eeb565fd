// kernels_expert.hip -- expert FFN stages of the W8A8 FP8 MoE layer on gfx950:
// gate/up grouped GEMM with the SiLU*up epilogue, per-row e4m3
// requantisation, down-projection grouped GEMM, and the weighted combine.
//
// "Routage MoE entre GPU": each expert is a feed-forward network with its
// own weights and only the selected experts process a token; the outputs are
// weighted, summed and put back in token order.  W8A8 FP8: Alpha-MoE article,
// opening section.
//
// Grouped GEMM schedule: weight-stationary, one workgroup per (work item,
// tile of output channels[, K split]).  A work item is an expert and up to
// 16*MSUB of its rows (16*ML with the two-shape kernel), so a decode-sized
// batch puts all of an expert's rows in one item and each active expert's
// weights cross HBM exactly once.
//
// Workgroup = W compute waves (1..8, chosen by the host) + 1 loader wave
// (2 for 256-row passes):
//  - the loader gathers the item's activation rows (e4m3) into a ring of four
//    LDS chunks with global_load_lds_dwordx4, three chunks ahead of the
//    compute waves (exact vmcnt waits, so only the chunk due next is waited
//    for), after one batch of row lookups; the rows' activation scales go to
//    an LDS table by direct-to-LDS dword loads issued ahead of the first
//    chunk;
//  - each compute wave streams NB weight operands of 16 rows (gate and up
//    rows of 16 channels, or 32 down channels) from HBM into registers
//    through a PF-deep prefetch ring, reads the activation fragments from LDS
//    (four row groups at a time) and runs v_mfma_f32_16x16x128_f8f6f4;
//  - one s_barrier per chunk hands buffers between them.  The compute side
//    waits only on LDS counters, so its weight prefetches stay in flight
//    across it.
//
// MFMA operand layout (same for A = activation rows and B = weight rows):
// lane l holds row l%16 and, of each 128-byte K step, the bytes
// [16*(l/16), +16) and [64 + 16*(l/16), +16).  Each 16-byte piece load of a
// wave then covers 16 rows x 64 contiguous bytes.  Result tile: lane l,
// element i = C[4*(l/16) + i][l%16].
#include "common.hpp"
#include "internal.hpp"
#include <stdlib.h>

#include "expert_dev.hpp"

namespace fp8moe {

// ------------------------------------------------------------------ grouped GEMM
// W compute waves + the loader wave(s).  With up to five compute waves and
// row passes of up to 128 rows two workgroups share a CU; otherwise one
// workgroup per CU (256-row passes use 130 KB of LDS and up to 256 VGPRs).
template <int MSUB, int NB, bool GATEUP, bool NT>
__global__ __launch_bounds__(MSUB > 8 || NB > 2 ? kGemmMaxThreadsWide : kGemmMaxThreads) void wsgemm_kernel(
    GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t abuf[Chunk<MSUB>::LDS];
  wsgemm_tile<MSUB, NB, GATEUP, NT>(g, blockIdx.x, abuf);
}

// Gate/up with the per-row requantisation fused into the epilogue: W compute
// waves of two weight operands (16 h channels each, W <= 12) span all
// f <= 192 channels of an item's rows, so the workgroup holds every h value
// of its rows and writes e4m3 codes and row scales instead of fp32 h.  Row
// passes of at most 64 rows keep 13 waves within 128 VGPRs each.
template <int MSUB, bool NT>
__global__ __launch_bounds__((kRqMaxWaves + 1) * 64) void wsgemm_rq_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t abuf[Chunk<MSUB>::LDS_RQ];
  wsgemm_tile<MSUB, 2, true, NT, true>(g, blockIdx.x, abuf);
}

// Prefill-sized batches: 256-row passes, eight waves that all gather and
// compute (one workgroup per CU: 256 VGPRs per wave, 66 KB of LDS).
// Workgroups are dealt to the eight XCDs in turn (workgroup i to XCD i % 8),
// and each XCD has its own L2: workgroup i takes the (item, tile) of its
// XCD's contiguous share of the blocks that have work, so an XCD runs the
// channel tiles of the same items (same activation rows) and the passes of
// the same expert (same weight tiles) side by side.  Measured at a
// 65536-row batch: L2 misses of the gate/up GEMM 2.4 GB -> 1.0 GB.
template <bool GATEUP, int O16>
__global__ __launch_bounds__(kPfWaves * 64) void pfgemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t abuf[PfChunk::LDS];
  int bid = blockIdx.x;
  if (g.rs.items) {
    const int N = GATEUP ? g.rs.f : g.rs.d;
    const int ch_wg = kPfWaves * (GATEUP ? 16 : 32);
    const int n_real = *g.rs.n_items * ((N + ch_wg - 1) / ch_wg) * g.splits;
    if (bid < n_real) {
      const int q = n_real >> 3, r = n_real & 7, x = bid & 7, j = bid >> 3;
      bid = x * q + min(x, r) + j;  // XCD x: blocks [x*q + min(x, r), +q + (x < r))
    }
  }
  pf_tile<GATEUP, O16>(g, bid, abuf);
}

// Two row-pass shapes in one launch.  Work items are cut at 16*ML rows; an
// item of at most 16*MS rows runs the MS shape (deeper weight prefetch, K
// steps batched per LDS chunk), a longer one the ML shape.  Routing that
// sends many of the batch's tokens to a few experts then still streams each
// of their weights once, and the common short items keep the faster shape.
// Both shapes have one loader wave and two weight operands per wave, hence
// the same tiling of the grid.
template <int MS, int ML, bool GATEUP, bool NT>
__global__ __launch_bounds__(kGemmMaxThreads) void wsgemm2_kernel(GemmArgs g) {
  static_assert(MS < ML && Chunk<ML>::LOADERS == 1, "two row-pass shapes, one loader wave");
  constexpr int LDS = Chunk<ML>::LDS > Chunk<MS>::LDS ? Chunk<ML>::LDS : Chunk<MS>::LDS;
  __shared__ __attribute__((aligned(1024))) uint8_t abuf[LDS];
  const int W = (int)(blockDim.x >> 6) - 1;
  const int N = GATEUP ? g.rs.f : g.rs.d;
  const int ch_wg = W * (GATEUP ? 16 : 32);
  const int n_tiles = (N + ch_wg - 1) / ch_wg;
  const int item_id = __builtin_amdgcn_readfirstlane((int)(blockIdx.x / g.splits) / n_tiles);
  int expert, row0, rows, real;
  if (!resolve_item(g.rs, item_id, expert, row0, rows, real)) return;
  if (__builtin_amdgcn_readfirstlane(rows) <= 16 * MS)
    wsgemm_tile<MS, 2, GATEUP, NT>(g, blockIdx.x, abuf);
  else
    wsgemm_tile<ML, 2, GATEUP, NT>(g, blockIdx.x, abuf);
}

// A-resident tiles (ares_tile): every wave computes; LDS sized at launch.
template <int MSUB>
constexpr int ares_pf() { return MSUB >= 8 ? 2 : 4; }

// At most eight waves (two per SIMD, up to 256 VGPRs each: the eight-row-group
// tiles need more than the 168 of nine waves).
template <int MSUB, bool GATEUP, bool NT>
__global__ __launch_bounds__(kAresMaxWaves * 64) void ares_kernel(GemmArgs g) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t ares_lds[];
  ares_tile<MSUB, GATEUP, NT, ares_pf<MSUB>()>(g, blockIdx.x, ares_lds);
}

template <bool GATEUP, bool NT>
static hipError_t launch_ares_t(const GemmArgs &g, int msub, int waves, hipStream_t stream) {
  const int N = GATEUP ? g.rs.f : g.rs.d;
  const int K = GATEUP ? g.rs.d : g.rs.f;
  const int ch_wg = waves * (GATEUP ? 16 : 32);
  const int n_tiles = (N + ch_wg - 1) / ch_wg;
  const int blocks = g.rs.max_items * ((n_tiles + g.ntg - 1) / g.ntg);
  if (blocks == 0) return hipSuccess;
  const int nks = (K + 127) / 128;
  const int scales = g.ntg * ch_wg * (GATEUP ? 2 : 1);
  auto go = [&](auto kern, int ms, int pf) {
    const int ksp = (nks + pf - 1) / pf * pf;
    kern<<<blocks, waves * 64, ares_lds_bytes(ms, ksp, scales), stream>>>(g);
    return hipGetLastError();
  };
  switch (msub) {
    case 1: return go(ares_kernel<1, GATEUP, NT>, 1, ares_pf<1>());
    case 2: return go(ares_kernel<2, GATEUP, NT>, 2, ares_pf<2>());
    case 4: return go(ares_kernel<4, GATEUP, NT>, 4, ares_pf<4>());
    case 8: return go(ares_kernel<8, GATEUP, NT>, 8, ares_pf<8>());
    default: return hipErrorInvalidValue;
  }
}

// LDS of the A block and row scales (the weight scales come on top, at most
// kAresScaleFloats of them).
static int32_t ares_lds_need(int32_t msub, int32_t K) {
  if (msub != 1 && msub != 2 && msub != 4 && msub != 8) return 1 << 30;
  const int pf = msub >= 8 ? 2 : 4;
  const int nks = (K + 127) / 128;
  return ares_lds_bytes(msub, (nks + pf - 1) / pf * pf, 0);
}

bool ares_fits(int32_t msub, int32_t K) {
  return K <= kAresMaxK && ares_lds_need(msub, K) + kAresScaleFloats * 4 <= kAresLdsMax;
}

hipError_t launch_ares(const RowSpace &rs, const uint8_t *a, const float *a_scale,
                       const ExpertWeights &w, float *out, _Float16 *out16, bool gate_up,
                       int32_t msub, int32_t waves, int32_t ntg, bool stream_weights,
                       hipStream_t stream) {
  if (!rs.items || !ares_fits(msub, gate_up ? rs.d : rs.f) || waves < 1 || waves > kAresMaxWaves ||
      ntg < 1 || ntg * waves * (gate_up ? 32 : 32) > kAresScaleFloats)
    return hipErrorInvalidValue;
  GemmArgs g{rs, a, a_scale, nullptr, w, out, 1, gate_up ? rs.d : rs.f};
  g.out16 = out16;
  g.ntg = ntg;
  if (gate_up)
    return stream_weights ? launch_ares_t<true, true>(g, msub, waves, stream)
                          : launch_ares_t<true, false>(g, msub, waves, stream);
  return stream_weights ? launch_ares_t<false, true>(g, msub, waves, stream)
                        : launch_ares_t<false, false>(g, msub, waves, stream);
}

__global__ __launch_bounds__(256) void down_f32_kernel(GemmArgs g) {
  down_f32_tile(g, blockIdx.x, threadIdx.x);
}

// ------------------------------------------------------------------ weight tile order
// Thread q writes bytes [16q, +16) of the tile-order matrix (moe_weights):
// tile q/128, half (q%128)/64, lane l = q%64 -> row 16*(tile/CT) + l%16,
// columns 128*(tile%CT) + 64*half + 16*(l/16) + [0, 16), zero past cols.
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint8_t *__restrict__ codes,
                                                           int rows, int cols,
                                                           uint8_t *__restrict__ packed) {
  const int CT = (cols + 127) >> 7;
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= (size_t)rows * CT * 8) return;
  const size_t tile = q >> 7;
  const int piece = (int)(q & 127), half = piece >> 6, l = piece & 63;
  const int r = (int)(tile / CT) * 16 + (l & 15);
  const int c = (int)(tile % CT) * 128 + half * 64 + (l >> 4) * 16;
  v4i v = {0, 0, 0, 0};
  if (c < cols) v = load16(codes + (size_t)r * cols + c);
  *reinterpret_cast<v4i *>(packed + q * 16) = v;
}

hipError_t launch_pack_weights(const uint8_t *codes, int32_t rows, int32_t cols, uint8_t *packed,
                               hipStream_t stream) {
  const size_t n = (size_t)rows * ((cols + 127) / 128) * 8;
  if (n == 0) return hipSuccess;
  pack_weights_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(codes, rows, cols, packed);
  return hipGetLastError();
}

// ------------------------------------------------------------------ requant
constexpr int kRowThreads = 256;

__global__ __launch_bounds__(kRowThreads) void requant_kernel(RowSpace rs, const float *__restrict__ h,
                                                              uint8_t *__restrict__ hq,
                                                              float *__restrict__ sh) {
  __shared__ float red[kRowThreads / kWave];
  requant_row<kRowThreads>(rs, h, hq, sh, blockIdx.x, red);
}

// ------------------------------------------------------------------ combine
template <typename Y>
__global__ __launch_bounds__(256) void combine_kernel(RowSpace rs, const Y *__restrict__ y,
                                                      int splits, const int32_t *__restrict__ ids,
                                                      const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv,
                                                      float *__restrict__ out) {
  combine_chunk<256>(rs, y, splits, ids, w, inv, out, blockIdx.x,
                     blockIdx.y * 256 * cols_per_load<Y>());
}

// fp16 y in one slab, 2048 columns of a token per workgroup.
__global__ __launch_bounds__(256) void combine_row_kernel(RowSpace rs, const _Float16 *__restrict__ y,
                                                          const int32_t *__restrict__ ids,
                                                          const float *__restrict__ w,
                                                          const int32_t *__restrict__ inv,
                                                          float *__restrict__ out) {
  combine_row16<256, 16>(rs, y, ids, w, inv, out, blockIdx.x, blockIdx.y * 256 * 8);
}

// ------------------------------------------------------------------ launchers

static int grid_items(const RowSpace &rs) { return rs.items ? rs.max_items : rs.E + rs.S; }

template <int MSUB, int NB, bool GATEUP, bool NT = false>
static hipError_t launch_ws(const GemmArgs &g, int waves, hipStream_t stream) {
  const int N = GATEUP ? g.rs.f : g.rs.d;
  const int ch_wave = GATEUP ? 8 * NB : 16 * NB;
  const int maxw = MSUB > 8 || NB > 2 ? kGemmMaxThreadsWide / 64 - Chunk<MSUB>::LOADERS : kGemmMaxWaves;
  const int wv = waves < 1 ? 1 : waves > maxw ? maxw : waves;
  const int n_tiles = (N + wv * ch_wave - 1) / (wv * ch_wave);
  const int blocks = grid_items(g.rs) * n_tiles * g.splits;
  if (blocks == 0) return hipSuccess;
  wsgemm_kernel<MSUB, NB, GATEUP, NT><<<blocks, (wv + Chunk<MSUB>::LOADERS) * 64, 0, stream>>>(g);
  return hipGetLastError();
}

template <bool GATEUP>
static hipError_t launch_pf(const GemmArgs &g, hipStream_t stream) {
  const int N = GATEUP ? g.rs.f : g.rs.d;
  const int ch_wg = kPfWaves * (GATEUP ? 16 : 32);
  const int n_tiles = (N + ch_wg - 1) / ch_wg;
  const int blocks = grid_items(g.rs) * n_tiles * g.splits;
  if (blocks == 0) return hipSuccess;
  if (g.out16)
    pfgemm_kernel<GATEUP, 1><<<blocks, kPfWaves * 64, 0, stream>>>(g);
  else
    pfgemm_kernel<GATEUP, 0><<<blocks, kPfWaves * 64, 0, stream>>>(g);
  return hipGetLastError();
}

template <int MS, int ML, bool GATEUP, bool NT>
static hipError_t launch_ws2(const GemmArgs &g, int waves, hipStream_t stream) {
  const int N = GATEUP ? g.rs.f : g.rs.d;
  const int ch_wave = GATEUP ? 16 : 32;
  const int wv = waves < 1 ? 1 : waves > kGemmMaxWaves ? kGemmMaxWaves : waves;
  const int n_tiles = (N + wv * ch_wave - 1) / (wv * ch_wave);
  const int blocks = grid_items(g.rs) * n_tiles * g.splits;
  if (blocks == 0) return hipSuccess;
  wsgemm2_kernel<MS, ML, GATEUP, NT><<<blocks, (wv + 1) * 64, 0, stream>>>(g);
  return hipGetLastError();
}

// The two-shape kernel for (msub, msub_big), or false when that pair has none.
template <bool GATEUP, bool NT>
static bool launch_pair(const GemmArgs &g, int msub, int msub_big, int waves, hipStream_t stream,
                        hipError_t *err) {
  switch (msub * 16 + msub_big) {
    case 1 * 16 + 2: *err = launch_ws2<1, 2, GATEUP, NT>(g, waves, stream); return true;
    case 1 * 16 + 4: *err = launch_ws2<1, 4, GATEUP, NT>(g, waves, stream); return true;
    case 1 * 16 + 8: *err = launch_ws2<1, 8, GATEUP, NT>(g, waves, stream); return true;
    case 2 * 16 + 4: *err = launch_ws2<2, 4, GATEUP, NT>(g, waves, stream); return true;
    case 2 * 16 + 8: *err = launch_ws2<2, 8, GATEUP, NT>(g, waves, stream); return true;
    case 4 * 16 + 8: *err = launch_ws2<4, 8, GATEUP, NT>(g, waves, stream); return true;
    default: return false;
  }
}

// Row passes of up to 128 rows with two weight operands per wave, with or
// without the non-temporal weight hint.
template <bool GATEUP, bool NT>
static hipError_t launch_nb2(const GemmArgs &g, int msub, int msub_big, int waves,
                             hipStream_t stream) {
  hipError_t err;
  if (launch_pair<GATEUP, NT>(g, msub, msub_big, waves, stream, &err)) return err;
  if (msub >= 8) return launch_ws<8, 2, GATEUP, NT>(g, waves, stream);
  if (msub >= 4) return launch_ws<4, 2, GATEUP, NT>(g, waves, stream);
  if (msub >= 2) return launch_ws<2, 2, GATEUP, NT>(g, waves, stream);
  return launch_ws<1, 2, GATEUP, NT>(g, waves, stream);
}

hipError_t launch_gate_up(const RowSpace &rs, const uint8_t *xq, const float *sx,
                          const ExpertWeights &w, float *h, int32_t msub, int32_t msub_big,
                          int32_t waves, int32_t nb, bool stream_weights, hipStream_t stream) {
  GemmArgs g{rs, xq, sx, nullptr, w, h, 1, rs.d};
  if (msub >= 16)
    return waves == kPfWaves ? launch_pf<true>(g, stream) : launch_ws<16, 2, true>(g, waves, stream);
  if (nb >= 4) {
    if (msub >= 8) return launch_ws<8, 4, true>(g, waves, stream);
    if (msub >= 4) return launch_ws<4, 4, true>(g, waves, stream);
    if (msub >= 2) return launch_ws<2, 4, true>(g, waves, stream);
    return launch_ws<1, 4, true>(g, waves, stream);
  }
  return stream_weights ? launch_nb2<true, true>(g, msub, msub_big, waves, stream)
                        : launch_nb2<true, false>(g, msub, msub_big, waves, stream);
}

template <int MSUB>
static hipError_t launch_rq_t(const GemmArgs &g, int waves, bool nt, hipStream_t stream) {
  const int blocks = grid_items(g.rs);  // one tile: the workgroup spans f
  if (blocks == 0) return hipSuccess;
  if (nt)
    wsgemm_rq_kernel<MSUB, true><<<blocks, (waves + 1) * 64, 0, stream>>>(g);
  else
    wsgemm_rq_kernel<MSUB, false><<<blocks, (waves + 1) * 64, 0, stream>>>(g);
  return hipGetLastError();
}

hipError_t launch_gate_up_rq(const RowSpace &rs, const uint8_t *xq, const float *sx,
                             const ExpertWeights &w, uint8_t *hq, float *sh, int32_t msub,
                             int32_t waves, bool stream_weights, hipStream_t stream) {
  if (waves < 1 || waves > kRqMaxWaves || waves * 16 < rs.f || msub < 1)
    return hipErrorInvalidValue;  // the host plans only tiles that span f
  GemmArgs g{rs, xq, sx, nullptr, w, nullptr, 1, rs.d};
  g.hq = hq;
  g.hsc = sh;
  // an item longer than the pass takes several passes (each row's amax
  // still spans the workgroup's channels)
  if (msub >= 4) return launch_rq_t<4>(g, waves, stream_weights, stream);
  if (msub >= 2) return launch_rq_t<2>(g, waves, stream_weights, stream);
  return launch_rq_t<1>(g, waves, stream_weights, stream);
}

// Rows of up to 4096 values: a wave per row, four rows per workgroup.
__global__ __launch_bounds__(256) void requant_wave_kernel(RowSpace rs, const float *__restrict__ h,
                                                           uint8_t *__restrict__ hq,
                                                           float *__restrict__ sh) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rs.capacity + rs.S * rs.T) return;
  requant_row_wave<16>(rs, h, hq, sh, row, threadIdx.x & 63);
}

hipError_t launch_requant(const RowSpace &rs, const float *h, uint8_t *hq, float *sh,
                          hipStream_t stream) {
  const int rows_total = rs.capacity + rs.S * rs.T;
  if (rows_total == 0) return hipSuccess;
  if (rs.f <= 4096)
    requant_wave_kernel<<<(rows_total + 3) / 4, 256, 0, stream>>>(rs, h, hq, sh);
  else
    requant_kernel<<<rows_total, kRowThreads, 0, stream>>>(rs, h, hq, sh);
  return hipGetLastError();
}

void down_split_geometry(int32_t f, int32_t msub, int32_t requested, int32_t *splits,
                         int32_t *ksplit) {
  const int kc = split_granule(msub >= 16 ? 16 : msub >= 8 ? 8 : msub >= 4 ? 4 : msub >= 2 ? 2 : 1);
  const int nchunks = (f + kc - 1) / kc;
  const int s = requested < 1 ? 1 : (requested > nchunks ? nchunks : requested);
  *ksplit = ((nchunks + s - 1) / s) * kc;
  *splits = (f + *ksplit - 1) / *ksplit;
}

int32_t down_splits_used(int32_t f, int32_t msub, int32_t splits) {
  int32_t s, k;
  down_split_geometry(f, msub, splits, &s, &k);
  return s;
}

hipError_t launch_down(const RowSpace &rs, const uint8_t *hq, const float *sh, const float *h32,
                       const ExpertWeights &w, float *y, _Float16 *y16, int32_t msub,
                       int32_t msub_big, int32_t splits, int32_t waves, int32_t nb,
                       bool stream_weights, hipStream_t stream) {
  if (h32) {
    GemmArgs g{rs, nullptr, nullptr, h32, w, y, 1, rs.f};
    const int blocks = grid_items(rs) * ((rs.d + 63) >> 6);
    if (blocks == 0) return hipSuccess;
    down_f32_kernel<<<blocks, 256, 0, stream>>>(g);
    return hipGetLastError();
  }
  int32_t ksplit;
  down_split_geometry(rs.f, msub, splits, &splits, &ksplit);
  GemmArgs g{rs, hq, sh, nullptr, w, y, splits, ksplit};
  g.out16 = y16;
  // 128-row passes and up (one round of workgroups at decode sizes): rotated
  // K starts, measured 95.6 -> 89.9 us at a Mixtral-shaped T=256 batch (the
  // shorter passes of smaller batches measured a little slower with it)
  g.krot = (msub >= 8 && msub < 16) ? 7 : 0;
  // ksplit is a whole number of msub chunks, hence of msub_big chunks too
  if (msub >= 16)
    return waves == kPfWaves ? launch_pf<false>(g, stream) : launch_ws<16, 2, false>(g, waves, stream);
  if (nb >= 4) {
    if (msub >= 8) return launch_ws<8, 4, false>(g, waves, stream);
    if (msub >= 4) return launch_ws<4, 4, false>(g, waves, stream);
    if (msub >= 2) return launch_ws<2, 4, false>(g, waves, stream);
    return launch_ws<1, 4, false>(g, waves, stream);
  }
  return stream_weights ? launch_nb2<false, true>(g, msub, msub_big, waves, stream)
                        : launch_nb2<false, false>(g, msub, msub_big, waves, stream);
}

hipError_t launch_combine(const RowSpace &rs, const float *y, const _Float16 *y16, int32_t splits,
                          const int32_t *ids, const float *w, const int32_t *inv_pairs, float *out,
                          hipStream_t stream) {
  if (splits < 1 || splits > kMaxDownSplits) return hipErrorInvalidValue;
  if (rs.T == 0) return hipSuccess;
  // one fp16 slab: 16-byte row pieces, a token's 2048 columns per workgroup
  // (prefill-sized batches measured 27-33 % faster than four columns per
  // thread -- DeepSeek-shaped T=8192 95 -> 66 us -- decode sizes the same).
  // FP8MOE_COMBINE_ROW_T: the smallest batch that takes it (tile tuning, tests).
  const char *row_env = getenv("FP8MOE_COMBINE_ROW_T");
  const int row_min_t = (row_env && *row_env) ? atoi(row_env) : 1;
  if (y16 && splits == 1 && rs.T >= row_min_t)
    combine_row_kernel<<<dim3(rs.T, (rs.d + 2047) / 2048), 256, 0, stream>>>(rs, y16, ids, w,
                                                                            inv_pairs, out);
  else if (y16)
    combine_kernel<_Float16><<<dim3(rs.T, (rs.d + 1023) / 1024), 256, 0, stream>>>(
        rs, y16, splits, ids, w, inv_pairs, out);
  else
    combine_kernel<float><<<dim3(rs.T, (rs.d + 1023) / 1024), 256, 0, stream>>>(
        rs, y, splits, ids, w, inv_pairs, out);
  return hipGetLastError();
}

// Debug build: this file's device-check word (see common.hpp).
FP8MOE_DEBUG_TAKE(expert)

}  // namespace fp8moe
