// kernels_permute.hip -- the permutation (dispatch on one device) as one
// 16-wave workgroup; the algorithm is in permute_dev.hpp.
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

int32_t max_work_items(int32_t T, int32_t E, int32_t k_max, int32_t block_m, int32_t n_shared,
                       int32_t row_chunk) {
  const int64_t cap = (int64_t)T * k_max + (int64_t)E * (block_m - 1);
  // sum_e ceil(pad_e / chunk) <= cap / chunk + E
  const int64_t routed = cap / row_chunk + E;
  const int64_t shared = (int64_t)n_shared * ((T + row_chunk - 1) / row_chunk);
  return (int32_t)(routed + shared);
}

hipError_t launch_permute(const int32_t *ids, int32_t T, int32_t E, int32_t k_max, int32_t block_m,
                          int32_t capacity, int32_t *sorted_pairs, int32_t *expert_offsets,
                          int32_t *block_expert, int32_t *inv_pairs, int32_t *n_blocks,
                          WorkItem *items, int32_t *n_items, int32_t row_chunk, int32_t n_shared,
                          hipStream_t stream) {
  permute_kernel<<<1, kPermThreads, 0, stream>>>(ids, T * k_max, E, block_m, capacity, sorted_pairs,
                                                 expert_offsets, block_expert, inv_pairs, n_blocks,
                                                 items, n_items, row_chunk, T, n_shared);
  return hipGetLastError();
}

}  // namespace fp8moe
