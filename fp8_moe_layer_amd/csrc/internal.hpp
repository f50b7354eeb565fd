// internal.hpp -- launch interface between the C ABI layer and the gfx950 kernels.
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp8moe.h"

namespace fp8moe {

// Set the calling thread's error text (moe_last_error) and return `code`;
// ok_status clears it and returns MOE_OK.
moe_status fail_status(moe_status code, const char *fmt, ...);
moe_status ok_status();

// One unit of grouped-GEMM work: `rows` consecutive expert rows starting at
// `row0` of the expert-rows layout, all belonging to `expert` (e >= E means
// shared expert e - E).
struct WorkItem {
  int32_t expert;
  int32_t row0;
  int32_t rows;
  int32_t real;  // the first `real` rows hold (token, slot) pairs, the rest padding
};

struct ExpertWeights {
  const uint8_t *w_gate, *w_up, *w_down;
  const float *s_gate, *s_up, *s_down;
  const uint8_t *ws_gate, *ws_up, *ws_down;
  const float *ss_gate, *ss_up, *ss_down;
};

// Shape of the expert-row space shared by the expert stages.
struct RowSpace {
  int32_t T, d, f, E, S, k_max;
  int32_t capacity;      // routed rows (padded); shared rows follow
  const int32_t *sorted_pairs;    // [capacity]
  const int32_t *expert_offsets;  // [E+1]
  const WorkItem *items;          // nullable: one item per expert, all its rows
  const int32_t *n_items;         // device count of valid items (with items)
  int32_t max_items;              // grid bound (with items)
};

// Row-major e4m3 codes [rows][cols] -> tile order (moe_weights).
hipError_t launch_pack_weights(const uint8_t *codes, int32_t rows, int32_t cols, uint8_t *packed,
                               hipStream_t stream);
hipError_t launch_quantize_rows(const float *x, int32_t rows, int32_t cols, uint8_t *q,
                                float *scale, hipStream_t stream);
hipError_t launch_router(const float *x, const float *w_router, const float *bias, int32_t T,
                         int32_t d, int32_t E, float *logits, hipStream_t stream);
// Router logits plus (xq != nullptr) the per-token quantisation of x, fused
// into one launch for decode-sized T*E.
constexpr int64_t kRouterDotMax = 1 << 16;
hipError_t launch_route_logits(const float *x, const float *w_router, const float *bias, int32_t T,
                               int32_t d, int32_t E, float *logits, uint8_t *xq, float *sx,
                               hipStream_t stream);
// Router logits + quantisation of x + top-k in one launch (decode-sized
// batches: route_fused_applies(T, E)); the logits equal launch_router's.
bool route_fused_applies(int32_t T, int32_t E);
hipError_t launch_route_topk_fused(const float *x, const float *w_router, const float *bias,
                                   int32_t T, int32_t d, int32_t E, int32_t k_max,
                                   const int32_t *kpt, float *logits, uint8_t *xq, float *sx,
                                   int32_t *ids, float *w, hipStream_t stream);
// Prefill-sized batches with E <= 128 (route_tile_applies(T, E)): logits,
// quantised x and top-k in one launch; the logits equal launch_router's.
bool route_tile_applies(int32_t T, int32_t E);
hipError_t launch_route_prefill(const float *x, const float *w_router, const float *bias,
                                int32_t T, int32_t d, int32_t E, int32_t k_max,
                                const int32_t *kpt, float *logits, uint8_t *xq, float *sx,
                                int32_t *ids, float *w, hipStream_t stream);
hipError_t launch_topk(const float *logits, int32_t T, int32_t E, int32_t k_max,
                       const int32_t *k_per_token, int32_t *ids, float *w, hipStream_t stream);
// items/n_items/row_chunk: optional work list for the expert stages (row_chunk
// rows per item); pass items == nullptr to skip it.
// counts: NULL, or permute_counts_ints(T, E, k_max) ints that nothing else
// writes while the work runs; with them a batch of four or more 1024-pair
// slices takes two launches instead of three (the same outputs).
int64_t permute_counts_ints(int32_t T, int32_t E, int32_t k_max);
hipError_t launch_permute(const int32_t *ids, int32_t T, int32_t E, int32_t k_max, int32_t block_m,
                          int32_t capacity, int32_t *sorted_pairs, int32_t *expert_offsets,
                          int32_t *block_expert, int32_t *inv_pairs, int32_t *n_blocks,
                          WorkItem *items, int32_t *n_items, int32_t row_chunk, int32_t n_shared,
                          hipStream_t stream, int32_t *counts = nullptr);
int32_t max_work_items(int32_t T, int32_t E, int32_t k_max, int32_t block_m, int32_t n_shared,
                       int32_t row_chunk);

// waves: compute waves per workgroup of the grouped GEMMs (1..8; with up to
// five, two workgroups share a CU).  With 256-row passes (msub 16), waves ==
// kPfWaves selects the prefill kernel (every wave gathers and computes),
// any other count the loader-wave kernel with that many computing waves.
constexpr int kGemmMaxWaves = 8;
constexpr int kGemmMaxThreads = (kGemmMaxWaves + 1) * 64;
// 256-row passes (msub 16, two loader waves) and four weight operands per
// wave (nb 4) use up to 256 VGPRs: at most eight waves per workgroup.
constexpr int kGemmMaxThreadsWide = 8 * 64;
constexpr int kGemmMaxWaves16 = 6;
constexpr int kPfWaves = 8;  // prefill GEMM: 256-row passes, every wave gathers and computes
// msub_big > msub (nb 2, msub_big <= 8): items longer than 16*msub rows run
// 16*msub_big-row passes in the same launch (items are cut at 16*msub_big).
// stream_weights (nb 2, msub <= 8): the weight loads carry the non-temporal
// hint -- for weights that one workgroup each reads once.
hipError_t launch_gate_up(const RowSpace &rs, const uint8_t *xq, const float *sx,
                          const ExpertWeights &w, float *h, int32_t msub, int32_t msub_big,
                          int32_t waves, int32_t nb, bool stream_weights, hipStream_t stream);
// Gate/up with the requantisation fused into its epilogue, for f <= 16 *
// kRqMaxWaves: one workgroup of `waves` two-operand compute waves (waves * 16
// >= f) per work item writes hq and sh (every row of the item) instead of h.
constexpr int kRqMaxWaves = 12;
hipError_t launch_gate_up_rq(const RowSpace &rs, const uint8_t *xq, const float *sx,
                             const ExpertWeights &w, uint8_t *hq, float *sh, int32_t msub,
                             int32_t waves, bool stream_weights, hipStream_t stream);
// Per-row e4m3 requantisation of h (real rows only): hq codes, sh = amax/448.
hipError_t launch_requant(const RowSpace &rs, const float *h, uint8_t *hq, float *sh,
                          hipStream_t stream);

// Debug build (FP8MOE_DEBUG): the device-check bits of each kernel file since
// the last call, after synchronising the device (bit 31: the read failed);
// always 0 in the release library.
uint32_t debug_take_route();
uint32_t debug_take_permute();
uint32_t debug_take_expert();
uint32_t debug_take_persistent();
// Down projection from hq/sh, or (h32 != nullptr) straight from fp32 h with
// fp32 products.  `splits` > 1 cuts K = f into that many ranges (fewer if f
// is short) whose partial sums go to separate y slabs [split][rows][d]; the
// count actually used is down_splits_used(f, msub, splits).  y16 (hq/sh
// input only): y written in fp16 there instead of fp32 to y.
hipError_t launch_down(const RowSpace &rs, const uint8_t *hq, const float *sh, const float *h32,
                       const ExpertWeights &w, float *y, _Float16 *y16, int32_t msub,
                       int32_t msub_big, int32_t splits, int32_t waves, int32_t nb,
                       bool stream_weights, hipStream_t stream);
int32_t down_splits_used(int32_t f, int32_t msub, int32_t splits);
// A-resident grouped GEMM (short K): the work items' activation rows for the
// whole K range in LDS, gathered once per workgroup; each workgroup of
// `waves` computing waves takes `ntg` consecutive N-tiles of its item; no K
// splits.  Applies when ares_fits(msub, K) (msub = the items' row passes,
// K <= kAresMaxK, the A block within the LDS budget); requires the work
// list.  Measured: it wins where K is a few steps and a workgroup takes
// several tiles (MoE-Prism-shaped down projection, K = 192: 131 -> 115 us);
// with K of 768 .. 2048 and one or two tiles per workgroup the per-tile
// kernels stay faster (the larger gather and LDS footprint cost more than
// the start-up latencies they save).
constexpr int kAresMaxK = 512;
constexpr int kAresMaxWaves = 8;       // waves per A-resident workgroup (all compute)
constexpr int kAresScaleFloats = 4096;  // weight scales staged per workgroup: ntg * waves * 32 at most
bool ares_fits(int32_t msub, int32_t K);
hipError_t launch_ares(const RowSpace &rs, const uint8_t *a, const float *a_scale,
                       const ExpertWeights &w, float *out, _Float16 *out16, bool gate_up,
                       int32_t msub, int32_t waves, int32_t ntg, bool stream_weights,
                       hipStream_t stream);
// Final K-split count and bytes per split for a requested split count.
void down_split_geometry(int32_t f, int32_t msub, int32_t requested, int32_t *splits,
                         int32_t *ksplit);
constexpr int kDownChannelsPerWave = 32;  // output channels per down-projection wave (nb 2)
constexpr int kMaxDownSplits = 8;         // K splits of the down projection (y slabs)
// out from y slabs summed in split order (splits <= kMaxDownSplits, else
// hipErrorInvalidValue); y16 != nullptr: the slabs are fp16 there.
hipError_t launch_combine(const RowSpace &rs, const float *y, const _Float16 *y16, int32_t splits,
                          const int32_t *ids, const float *w, const int32_t *inv_pairs, float *out,
                          hipStream_t stream);

// Everything the single-launch (persistent) layer needs: the same buffers
// as the per-stage path, plus the grid-barrier state (kPersistBarSlots
// words, kPersistBarStride words apart; word 0 is the status word: 0 = ok,
// 1 = a grid barrier timed out; the last slot holds workgroup 0's
// s_memrealtime stamps at the kernel's start, after each grid barrier and at
// its end, kPersistStamps of them).
constexpr int kPersistBarSlots = 35;
constexpr int kPersistStamps = 10;
constexpr int kPersistBarStride = 16384;  // 64 KB
constexpr size_t kPersistBarBytes = (size_t)kPersistBarSlots * kPersistBarStride * sizeof(uint32_t);
struct PersistentLaunch {
  RowSpace rs;  // with the work list (items cut at 16*msub rows)
  ExpertWeights w;
  const float *x, *w_router, *bias;
  const int32_t *kpt;
  const float *logits_override;
  float *logits;
  uint8_t *xq;
  float *sx;
  int32_t *ids;
  float *tw;
  int32_t *sorted, *offsets, *block_expert, *inv, *n_blocks;
  WorkItem *items;
  int32_t *n_items;
  float *h;
  uint8_t *hq;
  float *sh, *y, *out;
  _Float16 *y16;  // y in fp16 (requantised path), else nullptr
  uint32_t *bar;
  int32_t block_m, row_chunk, msub, splits, no_requant;
};
// Workgroups of the persistent grid for row passes of 16*msub rows (16: the
// prefill tile) on a device of `cus` compute units: one per compute unit, or
// 0 when the compiled kernel cannot keep one resident per compute unit.
int32_t persistent_grid(int32_t msub, int32_t cus);
// The barrier-state reset and the cooperative launch (grid from
// persistent_grid); returns the launch error.
hipError_t launch_persistent(const PersistentLaunch &p, int32_t grid, hipStream_t stream);

}  // namespace fp8moe
