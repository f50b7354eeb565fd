// batching.hip -- host-side grouping of a token pool into decode batches that
// activate few distinct routed experts (moe_group_tokens).
//
// "ELDR : Microsoft et KAIST accélèrent le décodage des MoE": every decode
// step loads the weights of each distinct expert its batch activates, so the
// step's cost follows the number of distinct experts D, and batches whose
// tokens share experts cost less; changing only which tokens share a batch
// leaves every token's output unchanged (tokens are independent).  The
// grouping below is this library's plain greedy reading of that idea: each
// batch starts from the lowest-numbered unplaced token and repeatedly takes
// the unplaced token that adds the fewest experts not yet in the batch
// (ties: the lowest token number).  Deterministic; O(n^2 + n*k) time.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "internal.hpp"

extern "C" moe_status moe_group_tokens(const int32_t *ids, int32_t n, int32_t k, int32_t E,
                                       int32_t batch, int32_t *order) {
  using fp8moe::fail_status;
  const char *fn = "moe_group_tokens";
  if (n < 0 || k < 1 || k > MOE_MAX_K || E < 1 || E > MOE_MAX_EXPERTS || batch < 1)
    return fail_status(MOE_ERR_SHAPE, "%s: n=%d k=%d E=%d batch=%d", fn, n, k, E, batch);
  if (n == 0) return fp8moe::ok_status();
  if (!ids || !order) return fail_status(MOE_ERR_NULL, "%s: ids and order are required", fn);
  for (int64_t i = 0; i < (int64_t)n * k; ++i)
    if (ids[i] < -1 || ids[i] >= E)
      return fail_status(MOE_ERR_SHAPE, "%s: ids[%lld]=%d outside [-1, E)", fn, (long long)i, ids[i]);

  // experts of each token (a slot of -1 is empty; a repeated id counts once)
  // and, per expert, the tokens that use it
  std::vector<int32_t> nx(n, 0), xs((size_t)n * k);
  std::vector<std::vector<int32_t>> users(E);
  for (int32_t t = 0; t < n; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = ids[(size_t)t * k + j];
      if (e < 0) continue;
      bool dup = false;
      for (int32_t q = 0; q < nx[t]; ++q) dup |= xs[(size_t)t * k + q] == e;
      if (dup) continue;
      xs[(size_t)t * k + nx[t]++] = e;
      users[e].push_back(t);
    }
  }

  std::vector<char> placed(n, 0), in_batch(E, 0);
  std::vector<int32_t> fresh(n);  // experts a token would add to the current batch
  int32_t done = 0, first = 0;
  while (done < n) {
    memset(in_batch.data(), 0, (size_t)E);
    for (int32_t t = 0; t < n; ++t) fresh[t] = nx[t];
    auto take = [&](int32_t t) {
      placed[t] = 1;
      order[done++] = t;
      for (int32_t q = 0; q < nx[t]; ++q) {
        const int32_t e = xs[(size_t)t * k + q];
        if (in_batch[e]) continue;
        in_batch[e] = 1;
        for (int32_t u : users[e]) --fresh[u];
      }
    };
    while (placed[first]) ++first;
    take(first);
    for (int32_t filled = 1; filled < batch && done < n; ++filled) {
      int32_t best = -1;
      for (int32_t t = first; t < n; ++t)
        if (!placed[t] && (best < 0 || fresh[t] < fresh[best])) best = t;
      take(best);
    }
  }
  return fp8moe::ok_status();
}

// Quality-tier batching of a pool by routing budget (moe_k_tiers).
//
// "MoE-Prism: Disentangling Monolithic Experts …", section Méthodologie B,
// offline (throughput-oriented) mode: requests are sorted by their routing
// budget k and grouped into tiers; a tier's residual batch is either
// dispatched at once or merged into the next tier, whose batches serve it at
// that tier's larger k (over-service), by a local throughput rule.  This
// library's reading of that rule: serving r residual tokens alone costs one
// batch overhead plus r*k_i (token, slot) pairs, merging them costs the
// r*(k_next - k_i) extra pairs they are over-served by, and the cheaper side
// wins (ties: dispatch, no over-service).  Tiers are taken in ascending k,
// tokens in ascending number; a merged residual leads the next tier's pool.
extern "C" moe_status moe_k_tiers(const int32_t *k_per_token, int32_t n, int32_t batch,
                                  int32_t overhead, int32_t *order, int32_t *batch_start,
                                  int32_t *batch_k, int32_t *n_batches) {
  using fp8moe::fail_status;
  const char *fn = "moe_k_tiers";
  if (n < 0 || batch < 1 || overhead < 0)
    return fail_status(MOE_ERR_SHAPE, "%s: n=%d batch=%d overhead=%d", fn, n, batch, overhead);
  if (!n_batches || !batch_start || (n > 0 && (!k_per_token || !order || !batch_k)))
    return fail_status(MOE_ERR_NULL, "%s: k_per_token, order, batch_start, batch_k and n_batches are required", fn);
  for (int32_t t = 0; t < n; ++t)
    if (k_per_token[t] < 1 || k_per_token[t] > MOE_MAX_K)
      return fail_status(MOE_ERR_SHAPE, "%s: k_per_token[%d]=%d outside [1, %d]", fn, t,
                         k_per_token[t], MOE_MAX_K);

  // tiers: the tokens of each budget, ascending
  std::vector<std::vector<int32_t>> tier(MOE_MAX_K + 1);
  for (int32_t t = 0; t < n; ++t) tier[k_per_token[t]].push_back(t);
  std::vector<int32_t> ks;
  for (int32_t k = 1; k <= MOE_MAX_K; ++k)
    if (!tier[k].empty()) ks.push_back(k);

  int32_t nb = 0, placed = 0;
  batch_start[0] = 0;
  auto dispatch = [&](const int32_t *toks, int32_t cnt, int32_t k) {
    for (int32_t i = 0; i < cnt; ++i) order[placed++] = toks[i];
    batch_k[nb] = k;
    batch_start[++nb] = placed;
  };
  std::vector<int32_t> pool;
  for (size_t i = 0; i < ks.size(); ++i) {
    const int32_t k = ks[i];
    pool.insert(pool.end(), tier[k].begin(), tier[k].end());  // carried residual first
    const int32_t full = (int32_t)pool.size() / batch * batch;
    for (int32_t b = 0; b < full; b += batch) dispatch(pool.data() + b, batch, k);
    const int32_t r = (int32_t)pool.size() - full;
    bool merge = false;
    if (r > 0 && i + 1 < ks.size()) {
      const int64_t alone = (int64_t)overhead + (int64_t)r * k, merged = (int64_t)r * ks[i + 1];
      merge = merged < alone;
    }
    if (r > 0 && !merge) dispatch(pool.data() + full, r, k);
    pool.erase(pool.begin(), pool.begin() + (merge ? full : full + r));
  }
  *n_batches = nb;
  return fp8moe::ok_status();
}
