// kernels_persistent.hip -- the whole W8A8 FP8 MoE layer forward in one
// cooperative launch on gfx950.  SWITCHED OFF: moe_fused_forward refuses
// MOE_F_PERSISTENT and nothing calls launch_persistent.  Under test the
// launch first read stale workspace (with an arrival-counter barrier whose
// reset kernel and single-wave fence proved insufficient) and then, with the
// runtime's cooperative grid barrier, never completed; the cause is not
// established, so the code stays compiled but unreachable.
//
// The Alpha-MoE article (section "Comment fonctionne le megakernel") fuses
// routing, gating, expert compute and the output combine into one
// persistent kernel so that no launch separates the stages.  This kernel
// does the same with the stage device functions of the per-stage path: a
// resident grid (two 5-wave workgroups per CU, co-residency promised by the
// cooperative launch) walks each phase with a grid-stride loop and crosses
// a device-wide barrier between phases:
//
//   quantise x + router logits | top-k | permutation (workgroup 0) |
//   gate/up GEMM tiles | requantisation rows | down GEMM tiles | combine
//
// Between phases every wave publishes its own stores with a device-scope
// fence, the grid meets at the runtime's cooperative grid barrier, and every
// wave fences again so that no stale cached line survives into the next
// phase (a workgroup barrier alone does not wait for the other waves'
// stores to complete, and the workspace is read across XCDs).
#include <hip/hip_cooperative_groups.h>

#include <algorithm>

#include "common.hpp"
#include "expert_dev.hpp"
#include "internal.hpp"
#include "permute_dev.hpp"
#include "route_dev.hpp"

namespace fp8moe {

namespace {

constexpr int kPWaves = 5;  // 4 compute + 1 loader in the GEMM phases
constexpr int kPThreads = kPWaves * kWave;

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
  int32_t block_m, row_chunk, splits, ksplit;
};

__device__ __forceinline__ void grid_barrier() {
  __threadfence();  // this wave's stores are complete and written back
  cooperative_groups::this_grid().sync();
  __threadfence();  // this wave's later loads miss any stale line
}

}  // namespace

template <int MSUB>
__global__ __launch_bounds__(kPThreads, 3) void moe_persistent_kernel(PersistArgs a) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kGemmLdsBytes];
  static_assert(kGemmLdsBytes >= (int)sizeof(float) * kRouterTileLdsFloats, "router tile LDS");
  static_assert(kGemmLdsBytes >= (int)sizeof(int) * permute_lds_ints<kPWaves>(), "permute LDS");
  constexpr int VECX = (kMaxFfn + kPThreads * 4 - 1) / (kPThreads * 4);
  float *red = reinterpret_cast<float *>(lds);

  const RowSpace &rs = a.rs;
  const int G = gridDim.x, B = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int T = rs.T, d = rs.d, E = rs.E, K = rs.k_max;

  // ---- 1. quantise x, router logits
  if (a.logits_override || (int64_t)T * E > kRouterDotMax) {
    for (int t = B; t < T; t += G) {
      quantize_row_block<kPThreads, VECX>(a.x + (size_t)t * d, d, a.xq + (size_t)t * d, a.sx + t,
                                          red);
      __syncthreads();  // red is reused by the next row
    }
    if (!a.logits_override) {
      const int tt = (T + kRT - 1) / kRT, te = (E + kRE - 1) / kRE;
      float *xs = reinterpret_cast<float *>(lds);
      for (int tile = B; tile < tt * te; tile += G)
        router_tile(a.x, a.w_router, a.bias, T, d, E, a.logits, (tile / te) * kRT,
                    (tile % te) * kRE, xs, xs + kRT * kRS);
    }
  } else {
    for (int wid = B * kPWaves + wave; wid < T * E; wid += G * kPWaves) {
      const int t = wid / E;
      router_dot_wave(a.x, a.w_router, a.bias, d, E, a.logits, a.xq, a.sx, t, wid - t * E, lane);
    }
  }
  grid_barrier();

  // ---- 2. top-k and routing weights
  const float *lg = a.logits_override ? a.logits_override : a.logits;
  for (int t = B * kPWaves + wave; t < T; t += G * kPWaves)
    topk_token_wave(lg, T, E, K, a.kpt, a.ids, a.tw, t, lane);
  grid_barrier();

  // ---- 3. permutation and work list (one workgroup)
  if (B == 0)
    permute_block<kPWaves>(a.ids, T * K, E, a.block_m, rs.capacity, a.sorted, a.offsets,
                           a.block_expert, a.inv, a.n_blocks, a.items, a.n_items, a.row_chunk, T,
                           rs.S, reinterpret_cast<int *>(lds));
  grid_barrier();

  // ---- 4. gate/up grouped GEMM + SiLU*up
  {
    const GemmArgs g{rs, a.xq, a.sx, nullptr, a.w, a.h, 1, d};
    const int n = rs.max_items * (rs.f / 64);
    for (int b = B; b < n; b += G) wsgemm_tile<MSUB, 2, true>(g, b, lds);
  }
  grid_barrier();

  // ---- 5. per-row requantisation
  const int rows_total = rs.capacity + rs.S * T;
  for (int row = B; row < rows_total; row += G) {
    requant_row<kPThreads>(rs, a.h, a.hq, a.sh, row, red);
    __syncthreads();
  }
  grid_barrier();

  // ---- 6. down grouped GEMM (K splits into separate slabs)
  {
    const GemmArgs g{rs, a.hq, a.sh, nullptr, a.w, a.y, a.splits, a.ksplit};
    const int n = rs.max_items * ((d + 4 * kDownChannelsPerWave - 1) / (4 * kDownChannelsPerWave)) * a.splits;
    for (int b = B; b < n; b += G) wsgemm_tile<MSUB, 2, false>(g, b, lds);
  }
  grid_barrier();

  // ---- 7. weighted combine
  {
    const int chunk = kPThreads * 4;
    const int nc = (d + chunk - 1) / chunk;
    for (int task = B; task < T * nc; task += G)
      combine_chunk<kPThreads>(rs, a.y, a.splits, a.ids, a.tw, a.inv, a.out, task / nc,
                               (task % nc) * chunk);
  }
}

namespace {

template <int MSUB>
hipError_t launch_persistent_t(const PersistArgs &pa, hipStream_t stream) {
  static int per_cu[2] = {-1, -1};  // cached occupancy per device ordinal (0, 1) else queried
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int occ = dev < 2 ? per_cu[dev] : -1;
  if (occ < 0) {
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, moe_persistent_kernel<MSUB>, kPThreads, 0);
    if (e != hipSuccess) return e;
    if (dev < 2) per_cu[dev] = occ;
  }
  int cus = 0, lds_cu = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
  if (e != hipSuccess) return e;
  // never more workgroups per CU than its LDS holds, whatever the query said
  if (lds_cu > 0) occ = std::min(occ, lds_cu / kGemmLdsBytes);
  if (occ < 1) return hipErrorCooperativeLaunchTooLarge;
  const int grid = occ * cus;
  PersistArgs args = pa;
  void *params[] = {&args};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void *>(moe_persistent_kernel<MSUB>),
                                    dim3(grid), dim3(kPThreads), params, 0, stream);
}

}  // namespace

hipError_t launch_persistent(const PersistentLaunch &p, hipStream_t stream) {
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
  a.out = p.out;
  a.block_m = p.block_m;
  a.row_chunk = p.row_chunk;
  const int msub = p.msub;
  down_split_geometry(p.rs.f, msub, p.splits, &a.splits, &a.ksplit);
  if (msub >= 8) return launch_persistent_t<8>(a, stream);
  if (msub >= 4) return launch_persistent_t<4>(a, stream);
  if (msub >= 2) return launch_persistent_t<2>(a, stream);
  return launch_persistent_t<1>(a, stream);
}

}  // namespace fp8moe
