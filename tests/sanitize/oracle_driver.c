/* Runs every entry point of the CPU oracle (oracle/moe_oracle.h) on small
 * seeded layers, for a build with AddressSanitizer and UndefinedBehaviour-
 * Sanitizer: routed and shared experts, per-token k, a logits override, the
 * no-requant mode, one and two threads.  Checks that every call succeeds,
 * that the stage-by-stage path (quantise, router, top-k, permute, gate/up,
 * requantise, down, combine) gives the forward's output bit for bit, and that
 * the outputs are finite.  Prints "oracle driver ok" and exits 0 on success. */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/moe_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, in [0, 1) */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) / 9007199254740992.0;
}
static float normal(void) { /* Box-Muller */
  const double u = uniform() + 1e-12, v = uniform();
  return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static void fill(float *a, size_t n, float s) {
  for (size_t i = 0; i < n; ++i) a[i] = normal() * s;
}
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      exit(1);                                                     \
    }                                                              \
  } while (0)

static void one_layer(int T, int d, int f, int E, int k, int S, int bm, int elastic,
                      int no_requant, int override_logits, int nthreads) {
  oracle_dims dm = {T, d, f, E, k, S, bm, no_requant ? ORACLE_F_NO_REQUANT : 0u};
  float *x = malloc(sizeof(float) * T * d), *wr = malloc(sizeof(float) * E * d);
  float *bias = malloc(sizeof(float) * E);
  fill(x, (size_t)T * d, 1.0f);
  fill(wr, (size_t)E * d, 1.0f / sqrtf((float)d));
  fill(bias, E, 0.5f);
  int32_t *kpt = NULL;
  if (elastic) {
    kpt = malloc(sizeof(int32_t) * T);
    for (int t = 0; t < T; ++t) kpt[t] = 1 + (int)(uniform() * k);
  }
  /* expert weights: fp32 draws quantised per output channel with the oracle's own row quantiser */
  const int ne = E + S;
  uint8_t *wg = malloc((size_t)ne * f * d), *wu = malloc((size_t)ne * f * d), *wd = malloc((size_t)ne * d * f);
  float *sg = malloc(sizeof(float) * ne * f), *su = malloc(sizeof(float) * ne * f), *sd = malloc(sizeof(float) * ne * d);
  float *tmp = malloc(sizeof(float) * (size_t)(f > d ? f : d) * (f > d ? f : d));
  for (int e = 0; e < ne; ++e) {
    fill(tmp, (size_t)f * d, 1.0f / sqrtf((float)d));
    CHECK(moe_oracle_quantize_rows(tmp, f, d, wg + (size_t)e * f * d, sg + (size_t)e * f) == 0);
    fill(tmp, (size_t)f * d, 1.0f / sqrtf((float)d));
    CHECK(moe_oracle_quantize_rows(tmp, f, d, wu + (size_t)e * f * d, su + (size_t)e * f) == 0);
    fill(tmp, (size_t)d * f, 1.0f / sqrtf((float)f));
    CHECK(moe_oracle_quantize_rows(tmp, d, f, wd + (size_t)e * d * f, sd + (size_t)e * d) == 0);
  }
  oracle_weights w = {wg, wu, sg, su, wd, sd, NULL, NULL, NULL, NULL, NULL, NULL};
  if (S) {
    const size_t gu = (size_t)E * f * d, dn = (size_t)E * d * f;
    w.ws_gate = wg + gu; w.ws_up = wu + gu; w.ws_down = wd + dn;
    w.ss_gate = sg + (size_t)E * f; w.ss_up = su + (size_t)E * f; w.ss_down = sd + (size_t)E * d;
  }

  /* the whole layer */
  float *logits = malloc(sizeof(float) * T * E);
  CHECK(moe_oracle_router_logits(x, wr, bias, T, d, E, logits, nthreads) == 0);
  float *out = malloc(sizeof(float) * T * d), *tw = malloc(sizeof(float) * T * k);
  int32_t *ids = malloc(sizeof(int32_t) * T * k);
  CHECK(moe_oracle_forward(&dm, x, override_logits ? NULL : wr, override_logits ? NULL : bias, kpt, &w,
                           override_logits ? logits : NULL, out, ids, tw, nthreads) == 0);
  for (size_t i = 0; i < (size_t)T * d; ++i) CHECK(isfinite(out[i]));

  /* the same layer stage by stage */
  uint8_t *xq = malloc((size_t)T * d);
  float *sx = malloc(sizeof(float) * T);
  CHECK(moe_oracle_quantize_rows(x, T, d, xq, sx) == 0);
  int32_t *ids2 = malloc(sizeof(int32_t) * T * k);
  float *tw2 = malloc(sizeof(float) * T * k);
  CHECK(moe_oracle_route_topk(logits, T, E, k, kpt, ids2, tw2) == 0);
  CHECK(memcmp(ids, ids2, sizeof(int32_t) * T * k) == 0);
  CHECK(memcmp(tw, tw2, sizeof(float) * T * k) == 0);
  const int64_t cap = moe_oracle_capacity(T, E, k, bm);
  const int64_t rows = cap + (int64_t)S * T;
  int32_t *sp = malloc(sizeof(int32_t) * cap), *off = malloc(sizeof(int32_t) * (E + 1));
  int32_t *be = malloc(sizeof(int32_t) * ((cap + bm - 1) / bm + 1)), *inv = malloc(sizeof(int32_t) * T * k);
  int32_t nb = 0;
  CHECK(moe_oracle_permute(ids2, T, E, k, bm, (int32_t)cap, sp, off, be, inv, &nb) == 0);
  float *h = calloc((size_t)rows * f, sizeof(float));
  CHECK(moe_oracle_expert_gate_up(&dm, (int32_t)cap, xq, sx, sp, off, &w, h, nthreads) == 0);
  uint8_t *hq = calloc((size_t)rows * f, 1);
  float *sh = calloc((size_t)rows, sizeof(float));
  if (!no_requant) CHECK(moe_oracle_quantize_rows(h, (int32_t)rows, f, hq, sh) == 0);
  float *y = calloc((size_t)rows * d, sizeof(float));
  CHECK(moe_oracle_expert_down(&dm, (int32_t)cap, no_requant ? NULL : hq, no_requant ? NULL : sh,
                               no_requant ? h : NULL, sp, off, &w, y, nthreads) == 0);
  float *out2 = malloc(sizeof(float) * T * d);
  CHECK(moe_oracle_combine(&dm, (int32_t)cap, y, ids2, tw2, inv, out2) == 0);
  CHECK(memcmp(out, out2, sizeof(float) * T * d) == 0);

  free(x); free(wr); free(bias); free(kpt); free(wg); free(wu); free(wd); free(sg); free(su);
  free(sd); free(tmp); free(logits); free(out); free(tw); free(ids); free(xq); free(sx);
  free(ids2); free(tw2); free(sp); free(off); free(be); free(inv); free(h); free(hq); free(sh);
  free(y); free(out2);
}

int main(void) {
  /* codec: every code decodes, encodes back to itself (NaN codes aside) */
  for (int c = 0; c < 256; ++c) {
    const float v = moe_oracle_e4m3_decode((uint8_t)c);
    if (!isnan(v)) CHECK(moe_oracle_e4m3_encode(v) == (uint8_t)c || v == 0.0f);
  }
  uint32_t bad = 0;
  CHECK(moe_oracle_codec_selfcheck(0x3F000000ull, 0x3F000000ull + 4096, &bad, 2) == 0);
  /*        T   d    f    E  k  S  bm elastic norq override threads */
  one_layer(16, 64, 128, 8, 2, 0, 16, 0, 0, 0, 1);
  one_layer(37, 128, 192, 16, 4, 2, 16, 1, 0, 0, 2);
  one_layer(29, 64, 64, 12, 3, 1, 1, 1, 1, 0, 2);
  one_layer(20, 128, 128, 64, 8, 0, 32, 1, 0, 1, 1);
  one_layer(1, 64, 128, 4, 4, 1, 128, 0, 0, 0, 1);
  puts("oracle driver ok");
  return 0;
}
