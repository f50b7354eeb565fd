/* Runs the host-side code of the HIP library (include/fp8moe.h) that needs no
 * GPU, for a host-only build of the library with AddressSanitizer and
 * UndefinedBehaviourSanitizer: workspace sizing over a sweep of layer
 * shapes, the host validation of every entry point (each call below fails
 * validation, so nothing is enqueued and no device memory is touched), and
 * the host batching planners (moe_group_tokens, moe_k_tiers) on seeded
 * pools, whose outputs are checked for being permutations and for covering
 * each token's budget.  Prints "abi host driver ok" and exits 0 on success. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/fp8moe.h"

#define CHECK(c)                                                      \
  do {                                                                \
    if (!(c)) {                                                       \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      exit(1);                                                        \
    }                                                                 \
  } while (0)

static uint32_t g_state = 12345u;
static uint32_t next_u32(void) { /* xorshift32 */
  g_state ^= g_state << 13;
  g_state ^= g_state >> 17;
  g_state ^= g_state << 5;
  return g_state;
}

static void check_permutation(const int32_t *order, int n) {
  char *seen = calloc((size_t)n + 1, 1);
  for (int i = 0; i < n; ++i) {
    CHECK(order[i] >= 0 && order[i] < n && !seen[order[i]]);
    seen[order[i]] = 1;
  }
  free(seen);
}

int main(void) {
  CHECK(moe_abi_version() == FP8MOE_ABI_VERSION);
  for (int s = -1; s <= 8; ++s) CHECK(moe_status_str(s) != NULL);

  /* workspace sizing: valid shapes give a size, invalid ones 0 with a message */
  const int Ts[] = {1, 7, 64, 256, 4096, 8192};
  const int Es[] = {1, 8, 64, 128, 512};
  for (unsigned i = 0; i < sizeof Ts / sizeof Ts[0]; ++i)
    for (unsigned j = 0; j < sizeof Es / sizeof Es[0]; ++j)
      for (int flags = 0; flags < 4; ++flags) {
        const int E = Es[j], k = E < 8 ? E : 8;
        moe_dims d = {Ts[i], 2048, 768, E, k, (int)(i % 3), 16, (uint32_t)flags};
        CHECK(moe_capacity(d.T, d.E, d.k_max, d.block_m) >= (int64_t)d.T * d.k_max);
        (void)moe_workspace_bytes(&d);
      }
  moe_dims bad = {0, 2048, 768, 8, 2, 0, 16, 0};
  CHECK(moe_workspace_bytes(&bad) == 0 && strlen(moe_last_error()) > 0);
  CHECK(moe_workspace_bytes(NULL) == 0);

  /* host validation of the device entry points: every call fails before any HIP call */
  float *fake = (float *)(uintptr_t)0x10000;
  moe_dims d = {16, 256, 512, 8, 2, 0, 16, 0};
  moe_weights w;
  memset(&w, 0, sizeof w);
  CHECK(moe_fused_forward(&d, fake, fake, NULL, NULL, &w, NULL, fake, NULL, NULL, fake, 1 << 20,
                          NULL) == MOE_ERR_NULL);
  CHECK(moe_fused_forward(NULL, fake, fake, NULL, NULL, &w, NULL, fake, NULL, NULL, fake, 1 << 20,
                          NULL) == MOE_ERR_NULL);
  moe_dims fc = d;
  fc.flags = 1u << 2; /* MOE_F_FUSED_COMBINE: refused */
  CHECK(moe_fused_forward_noalloc(&fc, fake, fake, NULL, NULL, &w, NULL, fake, NULL, NULL, NULL) ==
        MOE_ERR_UNSUPPORTED);
  CHECK(moe_quantize_rows(NULL, 4, 64, NULL, NULL, NULL) == MOE_ERR_NULL);
  CHECK(moe_router_logits(fake, fake, NULL, 4, 63, 8, fake, NULL) == MOE_ERR_SHAPE);
  CHECK(moe_route_topk(fake, 4, 8, 9, NULL, (int32_t *)fake, fake, NULL) == MOE_ERR_SHAPE);
  CHECK(moe_permute((int32_t *)fake, 4, 8, 2, 16, 1, (int32_t *)fake, (int32_t *)fake,
                    (int32_t *)fake, (int32_t *)fake, (int32_t *)fake, NULL) == MOE_ERR_SHAPE);
  CHECK(moe_pack_weights(NULL, 16, 64, NULL, NULL) == MOE_ERR_NULL);
  CHECK(moe_packed_weight_bytes(15, 64) == 0 && moe_packed_weight_bytes(16, 192) == 16 * 256);

  /* batching planners on seeded pools */
  for (int trial = 0; trial < 40; ++trial) {
    const int n = 1 + (int)(next_u32() % 300), k = 1 + (int)(next_u32() % 8);
    const int E = k + (int)(next_u32() % 60), batch = 1 + (int)(next_u32() % 70);
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)n * k), *order = malloc(sizeof(int32_t) * n);
    for (int i = 0; i < n * k; ++i) ids[i] = (next_u32() % 9 == 0) ? -1 : (int32_t)(next_u32() % E);
    CHECK(moe_group_tokens(ids, n, k, E, batch, order) == MOE_OK);
    check_permutation(order, n);
    ids[0] = E; /* outside [-1, E): refused */
    CHECK(moe_group_tokens(ids, n, k, E, batch, order) == MOE_ERR_SHAPE);

    int32_t *kpt = malloc(sizeof(int32_t) * n), *start = malloc(sizeof(int32_t) * (n + 1));
    int32_t *bk = malloc(sizeof(int32_t) * n), nb = 0;
    for (int t = 0; t < n; ++t) kpt[t] = 1 << (next_u32() % 6);
    const int overhead = (int)(next_u32() % 5000);
    CHECK(moe_k_tiers(kpt, n, batch, overhead, order, start, bk, &nb) == MOE_OK);
    check_permutation(order, n);
    CHECK(nb >= 1 && nb <= n && start[0] == 0 && start[nb] == n);
    for (int b = 0; b < nb; ++b) {
      CHECK(start[b + 1] > start[b] && start[b + 1] - start[b] <= batch);
      for (int i = start[b]; i < start[b + 1]; ++i) CHECK(kpt[order[i]] <= bk[b]);
    }
    kpt[n - 1] = 33; /* a budget above MOE_MAX_K: refused */
    CHECK(moe_k_tiers(kpt, n, batch, overhead, order, start, bk, &nb) == MOE_ERR_SHAPE);
    free(ids); free(order); free(kpt); free(start); free(bk);
  }
  CHECK(moe_group_tokens(NULL, 0, 2, 8, 4, NULL) == MOE_OK);
  puts("abi host driver ok");
  return 0;
}
