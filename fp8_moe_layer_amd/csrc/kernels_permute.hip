// kernels_permute.hip -- the permutation (dispatch on one device): one
// 16-wave workgroup for decode-sized batches, three launches over slices of
// the pairs for large ones; the algorithm is in permute_dev.hpp.
#include "common.hpp"
#include "internal.hpp"
#include "permute_dev.hpp"

namespace fp8moe {

constexpr int kPermWaves = 16;
constexpr int kPermThreads = kPermWaves * kWave;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t *__restrict__ ids, int P, int E, int bm, int capacity,
    int32_t *__restrict__ sorted_pairs, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ block_expert, int32_t *__restrict__ inv_pairs,
    int32_t *__restrict__ n_blocks, WorkItem *__restrict__ items, int32_t *__restrict__ n_items,
    int row_chunk, int T, int S) {
  __shared__ int lds[permute_lds_ints<kPermWaves>()];
  permute_block<kPermWaves>(ids, P, E, bm, capacity, sorted_pairs, expert_offsets, block_expert,
                            inv_pairs, n_blocks, items, n_items, row_chunk, T, S, lds);
}

// ------------------------------------------------------------------ many workgroups
// Slice s's count of expert e goes to counts[s * stride + e]: into the
// slice's own inv_pairs range (stride kSlice) for the three-launch path, or
// into a workspace of its own (stride E) for the two-launch path.
__global__ __launch_bounds__(kSliceWaves * kWave) void permute_count_kernel(
    const int32_t *__restrict__ ids, int P, int E, int32_t *__restrict__ counts, int stride) {
  __shared__ int cnt[kSliceWaves * kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int b0, b1;
  slice_range(P, blockIdx.x, b0, b1);
  const int per = (b1 - b0 + kSliceWaves - 1) / kSliceWaves;
  const int w0 = min(b1, b0 + wave * per), w1 = min(b1, w0 + per);
  for (int e = lane; e < E; e += kWave) cnt[wave * E + e] = 0;  // this wave's row
  __builtin_amdgcn_wave_barrier();
  slice_count(ids, w0, w1, E, expert_bits(E), cnt + wave * E, lane);
  __syncthreads();
  for (int e = tid; e < E; e += kSliceWaves * kWave) {
    int c[kSliceWaves];
#pragma unroll
    for (int w = 0; w < kSliceWaves; ++w) c[w] = cnt[w * E + e];
    int t = 0;
#pragma unroll
    for (int w = 0; w < kSliceWaves; ++w) t += c[w];
    counts[blockIdx.x * stride + e] = t;  // this slice's count of expert e
  }
}

constexpr int kLayoutRegSlices = 16;  // slices per thread held in registers

__global__ __launch_bounds__(1024) void permute_layout_kernel(
    int P, int E, int bm, int capacity, int32_t *__restrict__ sorted_pairs,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ block_expert,
    int32_t *__restrict__ inv_pairs, int32_t *__restrict__ n_blocks, WorkItem *__restrict__ items,
    int32_t *__restrict__ n_items, int row_chunk, int T, int S) {
  __shared__ int tot[kMaxExperts], off[kMaxExperts + 1], item_off[kMaxExperts + 1];
  __shared__ int part[1024];
  const int ns = permute_slices(P);
  // Exclusive prefix over the slices of each expert's counts, G threads per
  // expert: thread (g, e) sums the contiguous slices [s0, s1), the groups'
  // sums are prefixed in LDS, then each thread writes its slices' prefixes.
  // (One thread walking all slices waited one load latency per slice.)
  const int G = 1024 / E;
  const int per = (ns + G - 1) / G;
  const int e = threadIdx.x % E, g = threadIdx.x / E;
  const bool act = g < G;
  const int s0 = min(ns, g * per), s1 = min(ns, g * per + per);
  if (per <= kLayoutRegSlices) {
    // the thread's slice counts stay in registers: one read of them, and one
    // write of the slices' first rows once the segment offsets are known
    int c[kLayoutRegSlices];
    int sum = 0;
#pragma unroll
    for (int j = 0; j < kLayoutRegSlices; ++j) {
      c[j] = act && s0 + j < s1 ? inv_pairs[(s0 + j) * kSlice + e] : 0;
      sum += c[j];
    }
    if (act) part[g * E + e] = sum;
    __syncthreads();
    int run = 0;
    if (act) {
      for (int h = 0; h < g; ++h) run += part[h * E + e];
      if (g == G - 1) tot[e] = run + sum;  // the last group ends at slice ns
    }
    __syncthreads();
    build_layout<1024>(tot, off, item_off, P, E, bm, capacity, sorted_pairs, expert_offsets,
                       block_expert, n_blocks, items, n_items, row_chunk, T, S);
    if (act) {
      run += off[e];
#pragma unroll
      for (int j = 0; j < kLayoutRegSlices; ++j) {
        if (s0 + j < s1) inv_pairs[(s0 + j) * kSlice + e] = run;  // first row of slice s0 + j
        run += c[j];
      }
    }
    return;
  }
  if (act) {
    int sum = 0;
#pragma unroll 4
    for (int b = s0; b < s1; ++b) sum += inv_pairs[b * kSlice + e];
    part[g * E + e] = sum;
  }
  __syncthreads();
  if (act) {
    int run = 0;
    for (int h = 0; h < g; ++h) run += part[h * E + e];
    for (int b = s0; b < s1; ++b) {
      const int c = inv_pairs[b * kSlice + e];
      inv_pairs[b * kSlice + e] = run;
      run += c;
    }
    if (g == G - 1) tot[e] = run;  // the last group ends at slice ns
  }
  __syncthreads();
  build_layout<1024>(tot, off, item_off, P, E, bm, capacity, sorted_pairs, expert_offsets,
                     block_expert, n_blocks, items, n_items, row_chunk, T, S);
  if (act)
    for (int b = s0; b < s1; ++b) inv_pairs[b * kSlice + e] += off[e];  // first row of slice b
}

__global__ __launch_bounds__(kSliceWaves * kWave) void permute_scatter_kernel(
    const int32_t *__restrict__ ids, int P, int E, int32_t *__restrict__ sorted_pairs,
    int32_t *__restrict__ inv_pairs) {
  __shared__ int cnt[kSliceWaves * kMaxExperts], base[kMaxExperts];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int b0, b1;
  slice_range(P, blockIdx.x, b0, b1);
  for (int e = tid; e < E; e += kSliceWaves * kWave) base[e] = inv_pairs[b0 + e];
  const int per = (b1 - b0 + kSliceWaves - 1) / kSliceWaves;
  const int w0 = min(b1, b0 + wave * per), w1 = min(b1, w0 + per);
  const int nbits = expert_bits(E);
  for (int e = lane; e < E; e += kWave) cnt[wave * E + e] = 0;  // this wave's row
  __builtin_amdgcn_wave_barrier();
  slice_count(ids, w0, w1, E, nbits, cnt + wave * E, lane);
  // the slice's bases are read (above) before its inv_pairs entries are written (scatter)
  __syncthreads();
  for (int e = tid; e < E; e += kSliceWaves * kWave) {
    int c[kSliceWaves];
#pragma unroll
    for (int w = 0; w < kSliceWaves; ++w) c[w] = cnt[w * E + e];
    int s = base[e];
#pragma unroll
    for (int w = 0; w < kSliceWaves; ++w) {
      cnt[w * E + e] = s;
      s += c[w];
    }
  }
  __syncthreads();
  slice_scatter(ids, w0, w1, E, nbits, cnt + wave * E, sorted_pairs, inv_pairs, lane);
}

constexpr int kManySlices = 4;  // at least this many slices: the multi-workgroup path

// Layout and scatter in one launch (after permute_count_kernel wrote every
// slice's counts to `counts`, a buffer nothing else writes): each slice's
// workgroup reads all the counts, forms the per-expert totals, the padded
// segment offsets and its own slice's first rows, writes its share of the
// layout arrays (workgroup 0 also the offsets and the work list) and
// scatters its slice -- the rows and arrays of the three-launch path,
// without the single-workgroup layout launch between count and scatter.
__global__ __launch_bounds__(kSliceWaves * kWave) void permute_layout_scatter_kernel(
    const int32_t *__restrict__ ids, int P, int E, int bm, int capacity,
    const int32_t *__restrict__ counts, int32_t *__restrict__ sorted_pairs,
    int32_t *__restrict__ expert_offsets, int32_t *__restrict__ block_expert,
    int32_t *__restrict__ inv_pairs, int32_t *__restrict__ n_blocks, WorkItem *__restrict__ items,
    int32_t *__restrict__ n_items, int row_chunk, int T, int S) {
  constexpr int NT = kSliceWaves * kWave;
  __shared__ int cnt[kSliceWaves * kMaxExperts], tot[kMaxExperts], base[kMaxExperts];
  __shared__ int off[kMaxExperts + 1], item_off[kMaxExperts + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int ns = permute_slices(P), me = blockIdx.x;
  // totals, and the counts of the slices before this one
  for (int e = tid; e < E; e += NT) {
    int t = 0, before = 0;
#pragma unroll 8
    for (int sl = 0; sl < ns; ++sl) {
      const int c = counts[sl * E + e];
      before += sl < me ? c : 0;
      t += c;
    }
    tot[e] = t;
    base[e] = before;
  }
  __syncthreads();
  layout_offsets<NT>(tot, off, item_off, E, bm, row_chunk);
  layout_write<NT>(tot, off, item_off, P, E, bm, capacity, sorted_pairs, expert_offsets,
                   block_expert, n_blocks, items, n_items, row_chunk, T, S, me, ns);
  // this slice: each wave's count, then rows from the slice's first row per expert
  int b0, b1;
  slice_range(P, me, b0, b1);
  const int per = (b1 - b0 + kSliceWaves - 1) / kSliceWaves;
  const int w0 = min(b1, b0 + wave * per), w1 = min(b1, w0 + per);
  const int nbits = expert_bits(E);
  for (int e = lane; e < E; e += kWave) cnt[wave * E + e] = 0;  // this wave's row
  __builtin_amdgcn_wave_barrier();
  slice_count(ids, w0, w1, E, nbits, cnt + wave * E, lane);
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int c[kSliceWaves];
#pragma unroll
    for (int w = 0; w < kSliceWaves; ++w) c[w] = cnt[w * E + e];
    int r = off[e] + base[e];
#pragma unroll
    for (int w = 0; w < kSliceWaves; ++w) {
      cnt[w * E + e] = r;
      r += c[w];
    }
  }
  __syncthreads();
  slice_scatter(ids, w0, w1, E, nbits, cnt + wave * E, sorted_pairs, inv_pairs, lane);
}

int32_t max_work_items(int32_t T, int32_t E, int32_t k_max, int32_t block_m, int32_t n_shared,
                       int32_t row_chunk) {
  const int64_t cap = (int64_t)T * k_max + (int64_t)E * (block_m - 1);
  // sum_e ceil(pad_e / chunk) <= cap / chunk + E
  const int64_t routed = cap / row_chunk + E;
  const int64_t shared = (int64_t)n_shared * ((T + row_chunk - 1) / row_chunk);
  return (int32_t)(routed + shared);
}

int64_t permute_counts_ints(int32_t T, int32_t E, int32_t k_max) {
  const int ns = permute_slices(T * k_max);
  return ns >= kManySlices ? (int64_t)ns * E : 0;
}

hipError_t launch_permute(const int32_t *ids, int32_t T, int32_t E, int32_t k_max, int32_t block_m,
                          int32_t capacity, int32_t *sorted_pairs, int32_t *expert_offsets,
                          int32_t *block_expert, int32_t *inv_pairs, int32_t *n_blocks,
                          WorkItem *items, int32_t *n_items, int32_t row_chunk, int32_t n_shared,
                          hipStream_t stream, int32_t *counts) {
  const int P = T * k_max;
  const int ns = permute_slices(P);
  if (ns >= kManySlices && counts) {
    permute_count_kernel<<<ns, kSliceWaves * kWave, 0, stream>>>(ids, P, E, counts, E);
    permute_layout_scatter_kernel<<<ns, kSliceWaves * kWave, 0, stream>>>(
        ids, P, E, block_m, capacity, counts, sorted_pairs, expert_offsets, block_expert,
        inv_pairs, n_blocks, items, n_items, row_chunk, T, n_shared);
    return hipGetLastError();
  }
  if (ns >= kManySlices) {
    permute_count_kernel<<<ns, kSliceWaves * kWave, 0, stream>>>(ids, P, E, inv_pairs, kSlice);
    permute_layout_kernel<<<1, 1024, 0, stream>>>(P, E, block_m, capacity, sorted_pairs,
                                                  expert_offsets, block_expert, inv_pairs, n_blocks,
                                                  items, n_items, row_chunk, T, n_shared);
    permute_scatter_kernel<<<ns, kSliceWaves * kWave, 0, stream>>>(ids, P, E, sorted_pairs,
                                                                   inv_pairs);
    return hipGetLastError();
  }
  permute_kernel<<<1, kPermThreads, 0, stream>>>(ids, P, E, block_m, capacity, sorted_pairs,
                                                 expert_offsets, block_expert, inv_pairs, n_blocks,
                                                 items, n_items, row_chunk, T, n_shared);
  return hipGetLastError();
}

// Debug build: this file's device-check word (see common.hpp).
FP8MOE_DEBUG_TAKE(permute)

}  // namespace fp8moe
