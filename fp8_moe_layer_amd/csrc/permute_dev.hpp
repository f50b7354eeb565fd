// permute_dev.hpp -- the deterministic expert-sorted permutation as a
// workgroup-level device function (NW waves), shared by the per-stage kernel
// and the persistent single-launch kernel.
//
// "Routage MoE entre GPU": each token's activation is moved to the experts
// it selected, and at the end the weighted outputs are put back in the
// original token order.  On one device that movement is a grouping of the
// (token, slot) pairs by expert, padded to the GEMM row tile, plus the
// inverse map used by the combine.
//
// Each wave owns a contiguous slice of the pairs and walks it 64 at a time;
// lanes holding the same expert find each other with one ballot per
// expert-id bit, so a pair's rank among equal experts before it in the slice
// comes from a popcount, never from an atomic ticket.  Pass 1 counts per
// (wave, expert); a prefix over waves and an exclusive scan over the padded
// per-expert totals give every pair its row; pass 2 repeats the walk and
// scatters.  The order inside a segment is therefore ascending pair index,
// and the result is unique.
#pragma once
#include "common.hpp"
#include "internal.hpp"

namespace fp8moe {

constexpr int kBatch = 8;  // walk steps whose ids are loaded together

template <int NW>
constexpr int permute_lds_ints() {
  return NW * kMaxExperts + kMaxExperts + 2 * (kMaxExperts + 1);
}

// Lanes (among `valid` ones) holding the same expert id as this lane.
__device__ __forceinline__ uint64_t same_expert_mask(int e, bool valid, int nbits) {
  uint64_t m = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bb = __ballot(bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

// Pass 1 over one wave's slice [b0, b1): adds each expert's count to my[e].
__device__ __forceinline__ void slice_count(const int32_t *__restrict__ ids, int b0, int b1,
                                            int E, int nbits, int *my, int lane) {
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the slice's ids are fetched kBatch steps at a time so the loads overlap
  for (int base = b0; base < b1; base += kWave * kBatch) {
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = base + u * kWave + lane;
      ev[u] = p < b1 ? checked_id(ids[p], E) : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (base + u * kWave >= b1) break;  // uniform: the rest of the batch is past the slice
      const int e = ev[u];
      const bool valid = e >= 0;
      const uint64_t m = same_expert_mask(e, valid, nbits);
      if (valid && __popcll(m & lt_mask) == 0) my[e] += __popcll(m);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Pass 2 over the same slice: pair p of expert e goes to row my[e] + (its
// rank among the equal experts before it in the step); my[e] advances.
__device__ __forceinline__ void slice_scatter(const int32_t *__restrict__ ids, int b0, int b1,
                                              int E, int nbits, int *my, int32_t *__restrict__ sorted_pairs,
                                              int32_t *__restrict__ inv_pairs, int lane) {
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = b0; base < b1; base += kWave * kBatch) {
    int ev[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = base + u * kWave + lane;
      ev[u] = p < b1 ? checked_id(ids[p], E) : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (base + u * kWave >= b1) break;  // uniform
      const int p = base + u * kWave + lane;
      const int e = ev[u];
      const bool valid = e >= 0;
      const uint64_t m = same_expert_mask(e, valid, nbits);
      if (valid) {
        const int rank = __popcll(m & lt_mask);
        const int row = my[e] + rank;
        sorted_pairs[row] = p;
        inv_pairs[p] = row;
        // the leader's update is ordered after every lane's read above (same wave)
        __builtin_amdgcn_wave_barrier();
        if (rank == 0) my[e] += __popcll(m);
      } else if (p < b1) {
        inv_pairs[p] = -1;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

__device__ __forceinline__ int expert_bits(int E) {
  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

// From the per-expert totals tot[E] (LDS): padded segment offsets off[E+1]
// and work-list offsets item_off[E+1] (LDS).  Every thread of the workgroup
// calls this; it ends with a workgroup barrier.
template <int NT>
__device__ __forceinline__ void layout_offsets(const int *tot, int *off, int *item_off, int E,
                                               int bm, int row_chunk) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // exclusive scan of padded totals and of work-list offsets: lane l holds
  // experts [l*per, (l+1)*per), summed locally, then one wave scan
  if (wave == 0) {
    constexpr int PER = kMaxExperts / kWave;
    const int per = (E + kWave - 1) / kWave;
    const int e0 = lane * per;
    int pad[PER], ni[PER], ps = 0, is = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = e0 + j;
      const bool v = j < per && e < E;
      pad[j] = v ? (tot[e] + bm - 1) / bm * bm : 0;
      ni[j] = (v && row_chunk > 0) ? (pad[j] + row_chunk - 1) / row_chunk : 0;
      ps += pad[j];
      is += ni[j];
    }
    const int pinc = wave_incl_scan(ps, lane), iinc = wave_incl_scan(is, lane);
    int run = pinc - ps, irun = iinc - is;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = e0 + j;
      if (j < per && e < E) {
        off[e] = run;
        item_off[e] = irun;
      }
      run += pad[j];
      irun += ni[j];
    }
    if (lane == kWave - 1) {
      off[E] = pinc;
      item_off[E] = iinc;
    }
  }
  __syncthreads();
}

// The layout arrays from off / item_off / tot (LDS): part `part` of `parts`
// of the block table and of the padding sentinels; part 0 also writes
// expert_offsets, n_blocks and the work list.  No barrier.
template <int NT>
__device__ __forceinline__ void layout_write(const int *tot, const int *off, const int *item_off,
                                             int P, int E, int bm, int capacity,
                                             int32_t *__restrict__ sorted_pairs,
                                             int32_t *__restrict__ expert_offsets,
                                             int32_t *__restrict__ block_expert,
                                             int32_t *__restrict__ n_blocks,
                                             WorkItem *__restrict__ items,
                                             int32_t *__restrict__ n_items, int row_chunk, int T,
                                             int S, int part, int parts) {
  const int tid = threadIdx.x;
  const int sentinel = P;
  const int total = off[E];
  const int nb = total / bm;
  const int nb_cap = (capacity + bm - 1) / bm;
  auto range = [&](int n, int &lo, int &hi) {  // part's share of [0, n)
    lo = (int)((int64_t)n * part / parts);
    hi = (int)((int64_t)n * (part + 1) / parts);
  };
  int lo, hi;
  if (part == 0) {
    for (int e = tid; e <= E; e += NT) expert_offsets[e] = off[e];
    if (tid == 0) *n_blocks = nb;
  }
  // a thread per block: its expert is the last segment starting at or before
  // it (off is non-decreasing; empty segments start where the next one does)
  range(nb, lo, hi);
  for (int b = lo + tid; b < hi; b += NT) {
    const int row = b * bm;
    int l = 0, h = E - 1;  // off[l] <= row < off[E]
    while (l < h) {
      const int mid = (l + h + 1) >> 1;
      if (off[mid] <= row) l = mid;
      else h = mid - 1;
    }
    block_expert[b] = l;
  }
  range(E, lo, hi);
  for (int e = lo + tid; e < hi; e += NT)
    for (int r = off[e] + tot[e]; r < off[e + 1]; ++r) sorted_pairs[r] = sentinel;
  range(nb_cap - nb, lo, hi);
  for (int b = nb + lo + tid; b < nb + hi; b += NT) block_expert[b] = -1;
  range(capacity - total, lo, hi);
  for (int r = total + lo + tid; r < total + hi; r += NT) sorted_pairs[r] = sentinel;

  // work list for the expert stages: routed segments cut into row_chunk rows,
  // then the shared experts' token rows
  if (items && part == 0) {
    for (int e = tid; e < E; e += NT) {
      const int pad = off[e + 1] - off[e];
      int k = item_off[e];
      for (int r0 = 0; r0 < pad; r0 += row_chunk, ++k)
        items[k] = WorkItem{e, off[e] + r0, min(row_chunk, pad - r0),
                            max(0, min(row_chunk, tot[e] - r0))};
    }
    const int per_shared = (T + row_chunk - 1) / row_chunk;
    for (int i = tid; i < S * per_shared; i += NT) {
      const int s = i / per_shared, c = i % per_shared;
      const int r0 = c * row_chunk;
      const int rows = min(row_chunk, T - r0);
      items[item_off[E] + i] = WorkItem{E + s, capacity + s * T + r0, rows, rows};
    }
    if (tid == 0) *n_items = item_off[E] + S * per_shared;
  }
}

// The whole layout in one workgroup: offsets, then every array.  Every
// thread of the workgroup (NT of them) calls this; it ends with a workgroup
// barrier.
template <int NT>
__device__ __forceinline__ void build_layout(const int *tot, int *off, int *item_off, int P, int E,
                                             int bm, int capacity,
                                             int32_t *__restrict__ sorted_pairs,
                                             int32_t *__restrict__ expert_offsets,
                                             int32_t *__restrict__ block_expert,
                                             int32_t *__restrict__ n_blocks,
                                             WorkItem *__restrict__ items,
                                             int32_t *__restrict__ n_items, int row_chunk, int T,
                                             int S) {
  layout_offsets<NT>(tot, off, item_off, E, bm, row_chunk);
  layout_write<NT>(tot, off, item_off, P, E, bm, capacity, sorted_pairs, expert_offsets,
                   block_expert, n_blocks, items, n_items, row_chunk, T, S, 0, 1);
  __syncthreads();
}

// Every thread of the workgroup (NW waves) calls this; lds holds
// permute_lds_ints<NW>() ints.  items may be nullptr (no work list).
template <int NW>
__device__ __forceinline__ void permute_block(
    const int32_t *__restrict__ ids, int P, int E, int bm, int capacity,
    int32_t *__restrict__ sorted_pairs, int32_t *__restrict__ expert_offsets,
    int32_t *__restrict__ block_expert, int32_t *__restrict__ inv_pairs,
    int32_t *__restrict__ n_blocks, WorkItem *__restrict__ items, int32_t *__restrict__ n_items,
    int row_chunk, int T, int S, int *lds) {
  int *cnt = lds;                          // [NW][E] per (wave, expert) count, then base
  int *tot = cnt + NW * kMaxExperts;       // [E]
  int *off = tot + kMaxExperts;            // [E+1]
  int *item_off = off + kMaxExperts + 1;   // [E+1]
  constexpr int NT = NW * kWave;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nbits = expert_bits(E);

  // slices are whole 64-pair steps, so short batches leave the last waves idle
  const int per = (P + NW * kWave - 1) / (NW * kWave) * kWave;
  const int b0 = min(P, wave * per), b1 = min(P, b0 + per);
  int *my = cnt + wave * E;
  for (int e = lane; e < E; e += kWave) my[e] = 0;  // only this wave uses its row until the barrier
  __builtin_amdgcn_wave_barrier();
  slice_count(ids, b0, b1, E, nbits, my, lane);
  __syncthreads();

  // exclusive prefix over waves per expert (all NW counts read first); totals
  for (int e = tid; e < E; e += NT) {
    int c[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) c[w] = cnt[w * E + e];
    int s = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      cnt[w * E + e] = s;
      s += c[w];
    }
    tot[e] = s;
  }
  __syncthreads();
  build_layout<NT>(tot, off, item_off, P, E, bm, capacity, sorted_pairs, expert_offsets,
                   block_expert, n_blocks, items, n_items, row_chunk, T, S);

  // pass 2: scatter (rows from segment start + wave base + running count)
  for (int e = lane; e < E; e += kWave) my[e] += off[e];
  __builtin_amdgcn_wave_barrier();
  slice_scatter(ids, b0, b1, E, nbits, my, sorted_pairs, inv_pairs, lane);
}

// ------------------------------------------------------------------ many workgroups
// Large batches: the pairs are cut into slices of at least kSlice pairs (the
// last one takes the remainder), one 4-wave workgroup each.  Counting,
// then one workgroup scanning the slices' counts and laying out the
// segments, then the scatter -- the same rows as permute_block.  A slice's
// counts and then its base rows are kept in the first E entries of its own
// range of inv_pairs, which only its own workgroup overwrites, after reading
// them.
constexpr int kSlice = 1024;  // >= kMaxExperts: a slice's first E entries hold its counts
constexpr int kSliceWaves = 4;

__host__ __device__ inline int permute_slices(int P) { return P / kSlice; }

__device__ __forceinline__ void slice_range(int P, int blk, int &b0, int &b1) {
  const int ns = permute_slices(P);
  b0 = blk * kSlice;
  b1 = blk == ns - 1 ? P : b0 + kSlice;
}

}  // namespace fp8moe
