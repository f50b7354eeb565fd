// kernels_persistent.hip -- the whole W8A8 FP8 MoE layer forward in one
// resident-grid launch on gfx950 (MOE_F_PERSISTENT).
//
// The Alpha-MoE article (section "Comment fonctionne le megakernel") fuses
// routing, gating, expert compute and the output combine into one
// persistent kernel, so that no launch separates the stages.  This kernel
// runs the stage device functions of the per-stage path in one cooperative
// launch: one workgroup of eight waves per compute unit walks each phase
// with a grid-stride loop, and a grid-wide barrier separates the phases:
//
//   route (quantise x + logits [+ top-k]) | top-k | permutation |
//   gate/up GEMM tiles | requantisation rows | down GEMM tiles | combine
//
// Routing runs the same arithmetic as the per-stage kernels for the same
// batch shape, so logits, ids and weights are identical bit for bit.  The
// GEMM tiles are as wide as eight waves allow (the per-stage planner may
// choose narrower ones), so the down projection's rotated K start can differ
// and outputs agree with the per-stage path to rounding, not bit for bit.
//
// Grid barrier.  A workgroup arrives once all its waves' stores are
// complete (s_waitcnt) and its L2 has been written back (agent-scope release,
// buffer_wbl2); arrivals are counted in 16 group counters, the last of a
// group counts at a top counter (every counter on its own 64 KB, so the
// atomics of different groups go to different memory channels).  Leaving,
// the first workgroup of each XCD to see the barrier complete invalidates
// that XCD's L2 (agent-scope acquire) and publishes it; the others wait for
// that and invalidate their compute unit's L1.  One L2 invalidate per XCD
// instead of one per workgroup: measured on this chip, per-workgroup
// invalidates made a barrier of 256 workgroups take ~20 us.
//
// Every wait is bounded (s_memrealtime, 1 s).  A workgroup whose wait runs
// out sets the status word and leaves the kernel; every other workgroup
// then runs out at the next barrier it cannot pass, so the launch always
// ends, with status != 0 and the outputs invalid.  A grid that is not
// co-resident therefore fails instead of hanging (the cooperative launch
// refuses such a grid anyway).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "common.hpp"
#include "expert_dev.hpp"
#include "internal.hpp"
#include "permute_dev.hpp"
#include "route_dev.hpp"

namespace fp8moe {

namespace {

constexpr int kPWaves = 8;
constexpr int kPThreads = kPWaves * kWave;

// Barrier state: kBarSlots words kBarStride words apart (64 KB), zeroed by
// persistent_reset_kernel before every launch.
constexpr int kBarGroups = 16;
constexpr int kXcds = 8;
constexpr int kSlotStatus = 0, kSlotTop = 1, kSlotGroup = 2, kSlotXgen = kSlotGroup + kBarGroups,
              kSlotXrdy = kSlotXgen + kXcds, kSlotStamps = kSlotXrdy + kXcds;
constexpr uint64_t kBarTimeoutTicks = 100000000ull;  // 1 s of the 100 MHz s_memrealtime clock
static_assert(kSlotStamps + 1 <= kPersistBarSlots, "barrier slots");

__device__ __forceinline__ uint32_t *bar_slot(uint32_t *bar, int s) {
  return bar + (size_t)s * kPersistBarStride;
}

__device__ __forceinline__ uint32_t ld_agent(uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Waits until *p >= target; false when the deadline passes first.
__device__ __forceinline__ bool wait_ge(uint32_t *p, uint32_t target, uint64_t t0) {
  while (ld_agent(p) < target) {
    if (__builtin_amdgcn_s_memrealtime() - t0 > kBarTimeoutTicks) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Workgroup 0 records the 100 MHz clock at phase boundaries (stamp i).
__device__ __forceinline__ void stamp(uint32_t *bar, int i) {
  if (blockIdx.x == 0 && threadIdx.x == 0 && i < kPersistStamps)
    reinterpret_cast<uint64_t *>(bar_slot(bar, kSlotStamps))[i] = __builtin_amdgcn_s_memrealtime();
}

__device__ __forceinline__ uint32_t xcc_id() {
  // HW_REG_XCC_ID (20), bits [3:0]
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & (kXcds - 1);
}

// Barrier number gen (1, 2, ...) of the launch.  Returns false (uniformly in
// the workgroup) when a wait ran out or another workgroup already failed.
__device__ bool grid_barrier(uint32_t *bar, uint32_t gen, int *flag) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's loads and stores are complete
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // write back this XCD's L2
    const int G = gridDim.x;
    const int g = blockIdx.x % kBarGroups;
    const uint32_t ng = (uint32_t)(G / kBarGroups + (g < G % kBarGroups ? 1 : 0));
    const uint32_t groups = (uint32_t)min(G, kBarGroups);
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const uint32_t prev = __hip_atomic_fetch_add(bar_slot(bar, kSlotGroup + g), 1u,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev + 1 == ng * gen)
      __hip_atomic_fetch_add(bar_slot(bar, kSlotTop), 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    bool ok = wait_ge(bar_slot(bar, kSlotTop), groups * gen, t0);
    if (ok) {
      const uint32_t x = xcc_id();
      uint32_t expect = gen - 1;
      if (__hip_atomic_compare_exchange_strong(bar_slot(bar, kSlotXgen + x), &expect, gen,
                                               __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // invalidate this XCD's L2
        __hip_atomic_store(bar_slot(bar, kSlotXrdy + x), gen, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      } else {
        ok = wait_ge(bar_slot(bar, kSlotXrdy + x), gen, t0);
      }
    }
    if (ok && ld_agent(bar_slot(bar, kSlotStatus)) != 0) ok = false;
    if (!ok)
      __hip_atomic_store(bar_slot(bar, kSlotStatus), 1u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    *flag = ok;
  }
  __syncthreads();
  asm volatile("buffer_inv sc0" ::: "memory");  // this compute unit's L1
  return *flag != 0;
}

struct PersistArgs {
  RowSpace rs;  // with the work list
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
  _Float16 *y16;
  uint32_t *bar;
  int32_t block_m, row_chunk, splits, ksplit, krot;
  int32_t no_requant;
};

// LDS of the persistent workgroup: the largest phase (the routing tile of
// 128 experts, the GEMM rings, the permutation's tables).
constexpr int max3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
constexpr int kPLds = max3(route_tile_lds_bytes<128>(),
                           Chunk<8>::LDS > PfChunk::LDS ? Chunk<8>::LDS : PfChunk::LDS,
                           (int)sizeof(int) * permute_lds_ints<kPWaves>());

}  // namespace

// MS: row passes of 16*MS rows (MS <= 8), or PF: the prefill tile (256-row
// passes, every wave gathers and computes).
template <int MS, bool PF>
__global__ __launch_bounds__(kPThreads) void moe_persistent_kernel(PersistArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kPLds];
  __shared__ int flag;
  const RowSpace &rs = a.rs;
  const int G = gridDim.x, B = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int T = rs.T, d = rs.d, E = rs.E, K = rs.k_max;
  uint32_t gen = 0;
  stamp(a.bar, 0);

  // ---- route: logits (+ quantised x, + top-k) with the per-stage arithmetic
  const float *lg = a.logits_override ? a.logits_override : a.logits;
  bool topk_done = false;
  if (a.logits_override) {
    for (int t = B; t < T; t += G) {
      quantize_row_block<kPThreads, (MOE_MAX_HIDDEN + kPThreads * 4 - 1) / (kPThreads * 4)>(
          a.x + (size_t)t * d, d, a.xq + (size_t)t * d, a.sx + t, reinterpret_cast<float *>(lds));
      __syncthreads();
    }
  } else if ((int64_t)T * E <= kRouterDotMax) {
    for (int wid = B * kPWaves + wave; wid < T * E; wid += G * kPWaves) {
      const int t = wid / E;
      router_dot_wave(a.x, a.w_router, a.bias, d, E, a.logits, a.xq, a.sx, t, wid - t * E, lane);
    }
  } else {
    float *lf = reinterpret_cast<float *>(lds);
    if (E <= 32) {
      for (int b = B; b < (T + 63) / 64; b += G) {
        route_tile_block<32>(a.x, a.w_router, a.bias, T, d, E, K, a.kpt, a.logits, a.xq, a.sx,
                             a.ids, a.tw, b, 0, lf);
        __syncthreads();
      }
      topk_done = true;
    } else if (E <= 64) {
      for (int b = B; b < (T + 31) / 32; b += G) {
        route_tile_block<64>(a.x, a.w_router, a.bias, T, d, E, K, a.kpt, a.logits, a.xq, a.sx,
                             a.ids, a.tw, b, 0, lf);
        __syncthreads();
      }
      topk_done = true;
    } else {
      const int bx = (T + 15) / 16, by = (E + 127) / 128;
      for (int b = B; b < bx * by; b += G) {
        route_tile_block<128>(a.x, a.w_router, a.bias, T, d, E, K, a.kpt, a.logits, a.xq, a.sx,
                              E <= 128 ? a.ids : nullptr, a.tw, b % bx, b / bx, lf);
        __syncthreads();
      }
      topk_done = E <= 128;
    }
  }
  if (!grid_barrier(a.bar, ++gen, &flag)) return;
  stamp(a.bar, gen);

  // ---- top-k and routing weights
  if (!topk_done) {
    for (int t = B * kPWaves + wave; t < T; t += G * kPWaves)
      topk_token_wave(lg, T, E, K, a.kpt, a.ids, a.tw, t, lane);
    if (!grid_barrier(a.bar, ++gen, &flag)) return;
  stamp(a.bar, gen);
  }

  // ---- permutation and work list (one workgroup)
  if (B == 0)
    permute_block<kPWaves>(a.ids, T * K, E, a.block_m, rs.capacity, a.sorted, a.offsets,
                           a.block_expert, a.inv, a.n_blocks, a.items, a.n_items, a.row_chunk, T,
                           rs.S, reinterpret_cast<int *>(lds));
  if (!grid_barrier(a.bar, ++gen, &flag)) return;
  stamp(a.bar, gen);

  // ---- gate/up grouped GEMM + SiLU*up
  {
    const GemmArgs g{rs, a.xq, a.sx, nullptr, a.w, a.h, 1, d};
    if constexpr (PF) {
      const int n = rs.max_items * ((rs.f + kPfWaves * 16 - 1) / (kPfWaves * 16));
      for (int b = B; b < n; b += G) {
        pf_tile<true>(g, b, lds);
        __syncthreads();
      }
    } else {
      const int ch_wg = (kPWaves - 1) * 16;
      const int n = rs.max_items * ((rs.f + ch_wg - 1) / ch_wg);
      for (int b = B; b < n; b += G) {
        wsgemm_tile<MS, 2, true>(g, b, lds);
        __syncthreads();
      }
    }
  }
  if (!grid_barrier(a.bar, ++gen, &flag)) return;
  stamp(a.bar, gen);

  // ---- per-row requantisation of h
  const int rows_total = rs.capacity + rs.S * T;
  if (!a.no_requant) {
    if (rs.f <= 4096) {
      for (int row = B * kPWaves + wave; row < rows_total; row += G * kPWaves)
        requant_row_wave<16>(rs, a.h, a.hq, a.sh, row, lane);
    } else {
      for (int row = B; row < rows_total; row += G) {
        requant_row<kPThreads>(rs, a.h, a.hq, a.sh, row, reinterpret_cast<float *>(lds));
        __syncthreads();
      }
    }
    if (!grid_barrier(a.bar, ++gen, &flag)) return;
  stamp(a.bar, gen);
  }

  // ---- down grouped GEMM (K splits into separate slabs)
  if (a.no_requant) {
    const GemmArgs g{rs, nullptr, nullptr, a.h, a.w, a.y, 1, rs.f};
    const int n = rs.max_items * ((d + 63) >> 6);
    // two 256-thread halves take a tile each (no workgroup barriers inside)
    for (int b = 2 * B + (int)(threadIdx.x >> 8); b < n; b += 2 * G)
      down_f32_tile(g, b, threadIdx.x & 255);
  } else {
    GemmArgs g{rs, a.hq, a.sh, nullptr, a.w, a.y, a.splits, a.ksplit};
    g.krot = a.krot;
    g.out16 = a.y16;
    if constexpr (PF) {
      const int n = rs.max_items * ((d + kPfWaves * 32 - 1) / (kPfWaves * 32)) * a.splits;
      for (int b = B; b < n; b += G) {
        pf_tile<false, 1>(g, b, lds);  // the requantised path keeps y in fp16
        __syncthreads();
      }
    } else {
      const int ch_wg = (kPWaves - 1) * kDownChannelsPerWave;
      const int n = rs.max_items * ((d + ch_wg - 1) / ch_wg) * a.splits;
      for (int b = B; b < n; b += G) {
        wsgemm_tile<MS, 2, false>(g, b, lds);
        __syncthreads();
      }
    }
  }
  if (!grid_barrier(a.bar, ++gen, &flag)) return;
  stamp(a.bar, gen);

  // ---- weighted combine
  if (a.y16) {
    const int chunk = kPThreads * cols_per_load<_Float16>();
    const int nc = (d + chunk - 1) / chunk;
    for (int task = B; task < T * nc; task += G)
      combine_chunk<kPThreads>(rs, a.y16, a.splits, a.ids, a.tw, a.inv, a.out, task / nc,
                               (task % nc) * chunk);
  } else {
    const int chunk = kPThreads * cols_per_load<float>();
    const int nc = (d + chunk - 1) / chunk;
    for (int task = B; task < T * nc; task += G)
      combine_chunk<kPThreads>(rs, a.y, 1, a.ids, a.tw, a.inv, a.out, task / nc,
                               (task % nc) * chunk);
  }
  stamp(a.bar, kPersistStamps - 1);
}

// Zeroes the barrier state and the status word before a launch.
__global__ __launch_bounds__(64) void persistent_reset_kernel(uint32_t *bar) {
  if (threadIdx.x < kPersistBarSlots) bar[(size_t)threadIdx.x * kPersistBarStride] = 0;
}

namespace {

template <int MS, bool PF>
const void *kernel_of() {
  return reinterpret_cast<const void *>(moe_persistent_kernel<MS, PF>);
}

const void *persistent_kernel(int msub) {
  switch (msub) {
    case 1: return kernel_of<1, false>();
    case 2: return kernel_of<2, false>();
    case 4: return kernel_of<4, false>();
    case 8: return kernel_of<8, false>();
    case 16: return kernel_of<16, true>();
    default: return nullptr;
  }
}

}  // namespace

int32_t persistent_grid(int32_t msub, int32_t cus) {
  const void *fn = persistent_kernel(msub);
  if (!fn || cus < 1) return 0;
  // Co-residency from the compiled kernel's resources: one workgroup of
  // kPThreads threads per compute unit needs its LDS, its VGPRs for eight
  // waves (two per SIMD) and no more than that per CU.
  hipFuncAttributes at{};
  if (hipFuncGetAttributes(&at, fn) != hipSuccess) return 0;
  if (at.maxThreadsPerBlock < kPThreads) return 0;
  int dev = 0, lds_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
      hipSuccess)
    return 0;
  if (lds_cu > 0 && (size_t)lds_cu < at.sharedSizeBytes) return 0;
  int occ = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, fn, kPThreads, 0) != hipSuccess ||
      occ < 1)
    return 0;
  return cus;  // one workgroup per compute unit
}

hipError_t launch_persistent(const PersistentLaunch &p, int32_t grid, hipStream_t stream) {
  const void *fn = persistent_kernel(p.msub);
  if (!fn || grid < 1) return hipErrorInvalidValue;
  PersistArgs a{};
  a.rs = p.rs;
  a.w = p.w;
  a.x = p.x;
  a.w_router = p.w_router;
  a.bias = p.bias;
  a.kpt = p.kpt;
  a.logits_override = p.logits_override;
  a.logits = p.logits;
  a.xq = p.xq;
  a.sx = p.sx;
  a.ids = p.ids;
  a.tw = p.tw;
  a.sorted = p.sorted;
  a.offsets = p.offsets;
  a.block_expert = p.block_expert;
  a.inv = p.inv;
  a.n_blocks = p.n_blocks;
  a.items = p.items;
  a.n_items = p.n_items;
  a.h = p.h;
  a.hq = p.hq;
  a.sh = p.sh;
  a.y = p.y;
  a.y16 = p.y16;
  a.out = p.out;
  a.bar = p.bar;
  a.block_m = p.block_m;
  a.row_chunk = p.row_chunk;
  a.no_requant = p.no_requant;
  down_split_geometry(p.rs.f, p.msub, p.splits, &a.splits, &a.ksplit);
  a.krot = (p.msub >= 8 && p.msub < 16) ? 7 : 0;
  persistent_reset_kernel<<<1, 64, 0, stream>>>(p.bar);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  void *params[] = {&a};
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(kPThreads), params, 0, stream);
}

// Debug build: this file's device-check word (see common.hpp).
FP8MOE_DEBUG_TAKE(persistent)

}  // namespace fp8moe
