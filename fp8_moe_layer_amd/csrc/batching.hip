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
