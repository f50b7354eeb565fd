/*
 * moe_oracle.c -- CPU oracle for the W8A8 FP8 Mixture-of-Experts layer.
 *
 * TEST INFRASTRUCTURE ONLY: the plain, slow definition the GPU library is
 * checked against.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark load it.  It shares no code with the GPU library.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC -pthread.
 * Every reduction runs in fp32 in ascending index order; no FMA contraction,
 * so each step is exactly the sequence of IEEE operations written here.
 *
 * Sources for each step are named in the comment above it:
 *  - "Routage MoE entre GPU" (blog post): a router scores every expert for
 *    each token's hidden state, keeps the best k and emits one weight per
 *    pick; only those experts run; their outputs are multiplied by the
 *    weights, summed, and put back in the original token order.
 *  - Alpha-MoE article ("La nouvelle bibliotheque megakernel d'Aleph Alpha
 *    ...", opening section): 8-bit FP8 weights and 8-bit FP8 activations
 *    (W8A8).
 *  - The per-token activation scales, per-output-channel weight scales,
 *    SwiGLU expert form, e4m3 round-to-nearest-even, fp32 accumulation,
 *    tie-break by lower expert index, softmax over the selected logits,
 *    padding to the GEMM tile, shared experts and per-token k are the
 *    workload statement of this layer; where the pages leave a step open the
 *    reading taken is stated next to the step.
 */
#define _GNU_SOURCE
#include "moe_oracle.h"

#include <float.h>
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* threads: a dynamic parallel-for over [0, n)                               */
/* ------------------------------------------------------------------------ */

typedef void (*range_fn)(void *ctx, int64_t begin, int64_t end);

typedef struct {
  range_fn fn;
  void *ctx;
  int64_t n, chunk;
  int64_t next; /* shared cursor */
} pool_job;

static void *pool_worker(void *arg) {
  pool_job *j = (pool_job *)arg;
  for (;;) {
    int64_t b = __atomic_fetch_add(&j->next, j->chunk, __ATOMIC_RELAXED);
    if (b >= j->n) break;
    int64_t e = b + j->chunk < j->n ? b + j->chunk : j->n;
    j->fn(j->ctx, b, e);
  }
  return NULL;
}

static int resolve_threads(int n) {
  if (n > 0) return n;
  cpu_set_t set;
  CPU_ZERO(&set);
  if (sched_getaffinity(0, sizeof set, &set) == 0) {
    int c = CPU_COUNT(&set);
    if (c > 0) return c;
  }
  long c = sysconf(_SC_NPROCESSORS_ONLN);
  return c > 0 ? (int)c : 1;
}

static void parallel_for(int64_t n, int64_t chunk, int nthreads, range_fn fn, void *ctx) {
  if (n <= 0) return;
  nthreads = resolve_threads(nthreads);
  int64_t pieces = (n + chunk - 1) / chunk;
  if (nthreads > pieces) nthreads = (int)pieces;
  pool_job job = {fn, ctx, n, chunk, 0};
  if (nthreads <= 1) {
    fn(ctx, 0, n);
    return;
  }
  pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
  int started = 0;
  for (int i = 0; i < nthreads; ++i) {
    if (pthread_create(&tid[i], NULL, pool_worker, &job) != 0) break;
    ++started;
  }
  pool_worker(&job); /* the caller works too; also covers a failed create */
  for (int i = 0; i < started; ++i) pthread_join(tid[i], NULL);
  free(tid);
}

/* ------------------------------------------------------------------------ */
/* e4m3 (OCP E4M3FN) codec                                                   */
/* ------------------------------------------------------------------------ */

/* Value of every code, built from the format definition: sign bit, 4-bit
 * exponent with bias 7, 3-bit mantissa; exponent field 0 is subnormal
 * (m/8 * 2^-6); S.1111.111 is NaN; there are no infinities. */
static float g_dec[256];
static pthread_once_t g_dec_once = PTHREAD_ONCE_INIT;

static void build_decode_table(void) {
  for (int c = 0; c < 256; ++c) {
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 15 && m == 7)
      v = NAN;
    else if (e == 0)
      v = ldexpf((float)m, -9); /* (m/8) * 2^-6 */
    else
      v = ldexpf((float)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
    g_dec[c] = s ? -v : v;
  }
}

static inline const float *dec_table(void) {
  pthread_once(&g_dec_once, build_decode_table);
  return g_dec;
}

float moe_oracle_e4m3_decode(uint8_t c) { return dec_table()[c]; }

void moe_oracle_e4m3_decode_array(const uint8_t *c, int64_t n, float *out) {
  const float *t = dec_table();
  for (int64_t i = 0; i < n; ++i) out[i] = t[c[i]];
}

/* Round-to-nearest, ties to the even code, saturating: any |v| >= 448
 * (infinity included) becomes +-448; NaN stays NaN.  Works on the fp32 bit
 * pattern so that no intermediate rounding happens. */
uint8_t moe_oracle_e4m3_encode(float v) {
  uint32_t b;
  memcpy(&b, &v, sizeof b);
  uint8_t sign = (uint8_t)((b >> 24) & 0x80u);
  uint32_t a = b & 0x7fffffffu;
  if (a > 0x7f800000u) return (uint8_t)(sign | 0x7fu); /* NaN */
  if (a >= 0x43e00000u) return (uint8_t)(sign | 0x7eu); /* |v| >= 448 */
  if ((a >> 23) == 0) return sign;                       /* fp32 zero or subnormal (< 2^-126) */
  int32_t e32 = (int32_t)(a >> 23) - 127;
  uint32_t mant = a & 0x7fffffu;
  if (e32 >= -6) {
    /* normal e4m3 grid: keep the top 3 mantissa bits, round on the other 20;
     * a carry out of the mantissa correctly bumps the exponent field. */
    uint32_t q = ((uint32_t)(e32 + 7) << 3) | (mant >> 20);
    uint32_t rem = mant & 0xfffffu;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) q += 1;
    if (q > 0x7eu) q = 0x7eu; /* unreachable below 448, kept as the saturation rule */
    return (uint8_t)(sign | q);
  }
  /* subnormal e4m3 grid: multiples of 2^-9.  value = sig * 2^(e32-23), so
   * value / 2^-9 = sig >> (14 - e32).  q == 8 is the smallest normal code. */
  uint32_t sig = mant | 0x800000u;
  int shift = 14 - e32; /* >= 21 here */
  if (shift >= 25) return sign; /* value < 2^-10: rounds to zero */
  uint32_t q = sig >> shift;
  uint32_t rem = sig & ((1u << shift) - 1u);
  uint32_t half = 1u << (shift - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1;
  return (uint8_t)(sign | q);
}

void moe_oracle_e4m3_encode_array(const float *v, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = moe_oracle_e4m3_encode(v[i]);
}

/* Independent formulation used to pin the encoder: nearest finite value by
 * search over the value table (codes 0x00..0x7E are increasing), ties to the
 * code with an even mantissa, NaN to 0x7F, the sign copied. */
static uint8_t encode_by_search(float v) {
  const float *t = dec_table();
  uint32_t b;
  memcpy(&b, &v, sizeof b);
  uint8_t sign = (uint8_t)((b >> 24) & 0x80u);
  if (isnan(v)) return (uint8_t)(sign | 0x7fu);
  double av = fabs((double)v);
  int lo = 0, hi = 0x7e; /* largest code with value <= av */
  if (av >= (double)t[0x7e]) return (uint8_t)(sign | 0x7eu);
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if ((double)t[mid] <= av)
      lo = mid;
    else
      hi = mid - 1;
  }
  int c = lo;
  double dlo = av - (double)t[c], dhi = (double)t[c + 1] - av;
  if (dhi < dlo || (dhi == dlo && (c & 1))) c += 1;
  return (uint8_t)(sign | c);
}

typedef struct {
  uint64_t lo;
  int64_t bad;
  uint32_t first_bad;
  pthread_mutex_t mu;
} selfcheck_ctx;

static void selfcheck_range(void *p, int64_t b, int64_t e) {
  selfcheck_ctx *c = (selfcheck_ctx *)p;
  int64_t bad = 0;
  uint32_t first = 0xffffffffu;
  for (int64_t i = b; i < e; ++i) {
    uint32_t bits = (uint32_t)(c->lo + (uint64_t)i);
    float v;
    memcpy(&v, &bits, sizeof v);
    if (moe_oracle_e4m3_encode(v) != encode_by_search(v)) {
      if (bad == 0) first = bits;
      ++bad;
    }
  }
  if (bad) {
    pthread_mutex_lock(&c->mu);
    if (c->bad == 0 || first < c->first_bad) c->first_bad = first;
    c->bad += bad;
    pthread_mutex_unlock(&c->mu);
  }
}

int64_t moe_oracle_codec_selfcheck(uint64_t lo, uint64_t hi, uint32_t *first_bad, int nthreads) {
  if (hi > (1ull << 32)) hi = 1ull << 32;
  if (hi <= lo) return 0;
  selfcheck_ctx c;
  c.lo = lo;
  c.bad = 0;
  c.first_bad = 0;
  pthread_mutex_init(&c.mu, NULL);
  parallel_for((int64_t)(hi - lo), 1 << 20, nthreads, selfcheck_range, &c);
  pthread_mutex_destroy(&c.mu);
  if (first_bad) *first_bad = c.first_bad;
  return c.bad;
}

/* ------------------------------------------------------------------------ */
/* step 1: per-row e4m3 quantisation                                         */
/* ------------------------------------------------------------------------ */

/* One scale per row (per token for activations, per output channel for
 * weights): amax = max |x|; r = 448/amax, s = amax/448 (both one IEEE fp32
 * division); q = e4m3(x * r).  A zero row gets r = s = 1.  Dequantised value
 * is dec(q) * s. */
static void quantize_row(const float *x, int32_t cols, uint8_t *q, float *scale) {
  float amax = 0.0f;
  for (int32_t i = 0; i < cols; ++i) {
    float a = fabsf(x[i]);
    if (a > amax) amax = a;
  }
  float r = 1.0f, s = 1.0f;
  if (amax != 0.0f) {
    r = 448.0f / amax;
    s = amax / 448.0f;
  }
  for (int32_t i = 0; i < cols; ++i) q[i] = moe_oracle_e4m3_encode(x[i] * r);
  *scale = s;
}

static int all_finite(const float *x, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(x[i])) return 0;
  return 1;
}

int moe_oracle_quantize_rows(const float *x, int32_t rows, int32_t cols, uint8_t *q, float *scale) {
  if (!x || !q || !scale || rows < 0 || cols <= 0) return 1;
  if (!all_finite(x, (int64_t)rows * cols)) return 2;
  for (int32_t r = 0; r < rows; ++r)
    quantize_row(x + (int64_t)r * cols, cols, q + (int64_t)r * cols, scale + r);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* step 2: router logits (fp32, unquantised hidden state)                    */
/* ------------------------------------------------------------------------ */

/* The router reads each token's hidden state and scores every expert
 * ("Routage MoE entre GPU", the router paragraph): l[t,e] = x[t].W_r[e] (+ b[e]). */
typedef struct {
  const float *x, *w, *b;
  int32_t d, E;
  float *logits;
} router_ctx;

static void router_range(void *p, int64_t b, int64_t e) {
  router_ctx *c = (router_ctx *)p;
  for (int64_t t = b; t < e; ++t) {
    const float *xt = c->x + t * c->d;
    for (int32_t ex = 0; ex < c->E; ++ex) {
      const float *wr = c->w + (int64_t)ex * c->d;
      float acc = 0.0f;
      for (int32_t i = 0; i < c->d; ++i) acc += xt[i] * wr[i];
      if (c->b) acc += c->b[ex];
      c->logits[t * c->E + ex] = acc;
    }
  }
}

int moe_oracle_router_logits(const float *x, const float *w_router, const float *bias, int32_t T,
                             int32_t d, int32_t E, float *logits, int nthreads) {
  if (!x || !w_router || !logits || T < 0 || d <= 0 || E <= 0) return 1;
  router_ctx c = {x, w_router, bias, d, E, logits};
  parallel_for(T, 1, nthreads, router_range, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* step 3: top-k selection and routing weights                               */
/* ------------------------------------------------------------------------ */

/* Order all E experts by logit, largest first, equal logits by lower index
 * (a stable insertion sort on "strictly smaller moves back"; -0 == +0 as a
 * float comparison), keep the first k_t, and give them
 *   w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 * with the sum taken in slot order.  Slots k_t..k_max-1 get id -1 and w 0. */
static void topk_token(const float *l, int32_t E, int32_t k_max, int32_t kt, int32_t *order,
                       float *eps, int32_t *ids, float *w) {
  for (int32_t e = 0; e < E; ++e) order[e] = e;
  for (int32_t i = 1; i < E; ++i) {
    int32_t key = order[i];
    int32_t j = i - 1;
    while (j >= 0 && l[order[j]] < l[key]) {
      order[j + 1] = order[j];
      --j;
    }
    order[j + 1] = key;
  }
  float m = l[order[0]];
  float z = 0.0f;
  for (int32_t j = 0; j < kt; ++j) {
    eps[j] = expf(l[order[j]] - m);
    z += eps[j];
  }
  for (int32_t j = 0; j < k_max; ++j) {
    if (j < kt) {
      ids[j] = order[j];
      w[j] = eps[j] / z;
    } else {
      ids[j] = -1;
      w[j] = 0.0f;
    }
  }
}

int moe_oracle_route_topk(const float *logits, int32_t T, int32_t E, int32_t k_max,
                          const int32_t *k_per_token, int32_t *topk_ids, float *topk_w) {
  if (!logits || !topk_ids || !topk_w || T < 0 || E <= 0 || k_max < 1 || k_max > E) return 1;
  if (k_per_token)
    for (int32_t t = 0; t < T; ++t)
      if (k_per_token[t] < 1 || k_per_token[t] > k_max) return 2;
  if (!all_finite(logits, (int64_t)T * E)) return 3;
  int32_t *order = (int32_t *)malloc(sizeof(int32_t) * (size_t)E);
  float *eps = (float *)malloc(sizeof(float) * (size_t)k_max);
  for (int32_t t = 0; t < T; ++t) {
    int32_t kt = k_per_token ? k_per_token[t] : k_max;
    topk_token(logits + (int64_t)t * E, E, k_max, kt, order, eps, topk_ids + (int64_t)t * k_max,
               topk_w + (int64_t)t * k_max);
  }
  free(order);
  free(eps);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* step 4: dispatch = expert-sorted permutation padded to the tile           */
/* ------------------------------------------------------------------------ */

int64_t moe_oracle_capacity(int32_t T, int32_t E, int32_t k_max, int32_t block_m) {
  return (int64_t)T * k_max + (int64_t)E * (block_m - 1);
}

/* On one device, "moving each token's activation to its expert" (the
 * dispatch in "Routage MoE entre GPU") is a grouping of the (token, slot)
 * pairs by expert, and the inverse map is what "restores the original token
 * order" at the end.  Pair p = t*k_max + j is valid when ids[p] >= 0.
 * Expert e's segment starts at off[e] = sum_{e'<e} ceil(cnt[e']/bm)*bm and
 * holds its pairs in ascending p, then the sentinel T*k_max up to the padded
 * length; block_expert[b] names the expert of rows [b*bm, (b+1)*bm);
 * blocks past the last segment get -1; inv[p] is p's row (-1 if invalid). */
int moe_oracle_permute(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k_max,
                       int32_t block_m, int32_t capacity, int32_t *sorted_pairs,
                       int32_t *expert_offsets, int32_t *block_expert, int32_t *inv_pairs,
                       int32_t *n_blocks) {
  if (!topk_ids || !sorted_pairs || !expert_offsets || !block_expert || !inv_pairs || !n_blocks)
    return 1;
  if (T < 0 || E <= 0 || k_max < 1 || block_m < 1) return 1;
  if ((int64_t)capacity < moe_oracle_capacity(T, E, k_max, block_m)) return 2;
  int64_t P = (int64_t)T * k_max;
  int32_t sentinel = (int32_t)P;
  int64_t *cnt = (int64_t *)calloc((size_t)E, sizeof(int64_t));
  for (int64_t p = 0; p < P; ++p) {
    int32_t e = topk_ids[p];
    if (e < -1 || e >= E) {
      free(cnt);
      return 3;
    }
    if (e >= 0) cnt[e] += 1;
  }
  expert_offsets[0] = 0;
  for (int32_t e = 0; e < E; ++e) {
    int64_t padded = (cnt[e] + block_m - 1) / block_m * block_m;
    expert_offsets[e + 1] = expert_offsets[e] + (int32_t)padded;
  }
  for (int32_t r = 0; r < capacity; ++r) sorted_pairs[r] = sentinel;
  int64_t *fill = (int64_t *)malloc(sizeof(int64_t) * (size_t)E);
  for (int32_t e = 0; e < E; ++e) fill[e] = expert_offsets[e];
  for (int64_t p = 0; p < P; ++p) {
    int32_t e = topk_ids[p];
    if (e < 0) {
      inv_pairs[p] = -1;
      continue;
    }
    int64_t row = fill[e]++;
    sorted_pairs[row] = (int32_t)p;
    inv_pairs[p] = (int32_t)row;
  }
  int32_t nb = expert_offsets[E] / block_m;
  int32_t nb_cap = (capacity + block_m - 1) / block_m;
  for (int32_t b = 0; b < nb_cap; ++b) block_expert[b] = -1;
  for (int32_t e = 0; e < E; ++e)
    for (int32_t b = expert_offsets[e] / block_m; b < expert_offsets[e + 1] / block_m; ++b)
      block_expert[b] = e;
  *n_blocks = nb;
  free(cnt);
  free(fill);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* steps 5-7: one expert FFN row                                             */
/* ------------------------------------------------------------------------ */

/* Each expert is a feed-forward network with its own weights ("Routage MoE
 * entre GPU", the expert paragraph), here the SwiGLU form with fp8 weights
 * and activations.  For one (token, expert) row:
 *   G[o] = sum_i dec(xq[i]) * dec(Wg[o][i]),  g = (G * sx) * sg[o]
 *   U[o] likewise with W_up,                  u = (U * sx) * su[o]
 *   h[o] = (g / (1 + exp(-g))) * u                                          */
static void gate_up_row(const float *xv, float sx, const uint8_t *wg, const uint8_t *wu,
                        const float *sg, const float *su, int32_t d, int32_t f, float *h) {
  const float *t = dec_table();
  for (int32_t o = 0; o < f; ++o) {
    const uint8_t *rg = wg + (int64_t)o * d;
    const uint8_t *ru = wu + (int64_t)o * d;
    float G = 0.0f, U = 0.0f;
    for (int32_t i = 0; i < d; ++i) {
      G += xv[i] * t[rg[i]];
      U += xv[i] * t[ru[i]];
    }
    float g = (G * sx) * sg[o];
    float u = (U * sx) * su[o];
    h[o] = (g / (1.0f + expf(-g))) * u;
  }
}

/* Down projection for one row.  a[] is dec(hq) (requantised, scale sh) or h
 * itself (requantisation disabled, sh unused):
 *   Y[c] = sum_o a[o] * dec(Wd[c][o]),  y = (Y * sh) * sd[c]  or  Y * sd[c]  */
static void down_row(const float *a, float sh, int requant, const uint8_t *wd, const float *sd,
                     int32_t d, int32_t f, float *y) {
  const float *t = dec_table();
  for (int32_t c = 0; c < d; ++c) {
    const uint8_t *r = wd + (int64_t)c * f;
    float Y = 0.0f;
    for (int32_t o = 0; o < f; ++o) Y += a[o] * t[r[o]];
    y[c] = requant ? (Y * sh) * sd[c] : Y * sd[c];
  }
}

/* Weight pointers of expert ex: ex < E routed, ex >= E shared (ex - E). */
typedef struct {
  const uint8_t *wg, *wu, *wd;
  const float *sg, *su, *sd;
} expert_ptrs;

static expert_ptrs expert_at(const oracle_dims *dm, const oracle_weights *w, int32_t ex) {
  expert_ptrs p;
  int64_t fd = (int64_t)dm->f * dm->d;
  if (ex < dm->E) {
    p.wg = w->w_gate + ex * fd;
    p.wu = w->w_up + ex * fd;
    p.wd = w->w_down + ex * fd;
    p.sg = w->s_gate + (int64_t)ex * dm->f;
    p.su = w->s_up + (int64_t)ex * dm->f;
    p.sd = w->s_down + (int64_t)ex * dm->d;
  } else {
    int64_t s = ex - dm->E;
    p.wg = w->ws_gate + s * fd;
    p.wu = w->ws_up + s * fd;
    p.wd = w->ws_down + s * fd;
    p.sg = w->ss_gate + s * dm->f;
    p.su = w->ss_up + s * dm->f;
    p.sd = w->ss_down + s * dm->d;
  }
  return p;
}

static int check_dims(const oracle_dims *dm, const oracle_weights *w) {
  if (!dm || !w) return 1;
  if (dm->T < 0 || dm->d <= 0 || dm->f <= 0 || dm->E <= 0 || dm->k_max < 1 || dm->k_max > dm->E ||
      dm->n_shared < 0 || dm->block_m < 1)
    return 1;
  if (!w->w_gate || !w->w_up || !w->w_down || !w->s_gate || !w->s_up || !w->s_down) return 1;
  if (dm->n_shared > 0 &&
      (!w->ws_gate || !w->ws_up || !w->ws_down || !w->ss_gate || !w->ss_up || !w->ss_down))
    return 1;
  return 0;
}

/* Expert row r of the stage layout -> (expert, token), or expert -1 for a
 * padding row. */
static void row_owner(const oracle_dims *dm, int32_t capacity, const int32_t *sorted_pairs,
                      const int32_t *expert_offsets, int64_t r, int32_t *ex, int32_t *tok) {
  if (r >= capacity) {
    int64_t q = r - capacity;
    *ex = dm->E + (int32_t)(q / dm->T);
    *tok = (int32_t)(q % dm->T);
    return;
  }
  int32_t p = sorted_pairs[r];
  if (p == dm->T * dm->k_max) {
    *ex = -1;
    *tok = -1;
    return;
  }
  int32_t e = 0;
  while (!(r >= expert_offsets[e] && r < expert_offsets[e + 1])) ++e;
  *ex = e;
  *tok = p / dm->k_max;
}

typedef struct {
  const oracle_dims *dm;
  int32_t capacity;
  const uint8_t *xq;
  const float *sx;
  const uint8_t *hq;
  const float *sh;
  const float *h;
  const int32_t *sorted_pairs, *expert_offsets;
  const oracle_weights *w;
  float *out;
} stage_ctx;

static void gate_up_range(void *p, int64_t b, int64_t e) {
  stage_ctx *c = (stage_ctx *)p;
  const oracle_dims *dm = c->dm;
  float *xv = (float *)malloc(sizeof(float) * (size_t)dm->d);
  for (int64_t r = b; r < e; ++r) {
    int32_t ex, tok;
    row_owner(dm, c->capacity, c->sorted_pairs, c->expert_offsets, r, &ex, &tok);
    if (ex < 0) continue;
    expert_ptrs wp = expert_at(dm, c->w, ex);
    moe_oracle_e4m3_decode_array(c->xq + (int64_t)tok * dm->d, dm->d, xv);
    gate_up_row(xv, c->sx[tok], wp.wg, wp.wu, wp.sg, wp.su, dm->d, dm->f, c->out + r * dm->f);
  }
  free(xv);
}

int moe_oracle_expert_gate_up(const oracle_dims *dims, int32_t capacity, const uint8_t *xq,
                              const float *sx, const int32_t *sorted_pairs,
                              const int32_t *expert_offsets, const oracle_weights *w, float *h,
                              int nthreads) {
  if (check_dims(dims, w) || !xq || !sx || !sorted_pairs || !expert_offsets || !h) return 1;
  if ((int64_t)capacity < moe_oracle_capacity(dims->T, dims->E, dims->k_max, dims->block_m))
    return 2;
  stage_ctx c = {dims, capacity, xq, sx, NULL, NULL, NULL, sorted_pairs, expert_offsets, w, h};
  int64_t rows = (int64_t)capacity + (int64_t)dims->n_shared * dims->T;
  parallel_for(rows, 1, nthreads, gate_up_range, &c);
  return 0;
}

static void down_range(void *p, int64_t b, int64_t e) {
  stage_ctx *c = (stage_ctx *)p;
  const oracle_dims *dm = c->dm;
  int requant = !(dm->flags & ORACLE_F_NO_REQUANT);
  float *a = (float *)malloc(sizeof(float) * (size_t)dm->f);
  for (int64_t r = b; r < e; ++r) {
    int32_t ex, tok;
    row_owner(dm, c->capacity, c->sorted_pairs, c->expert_offsets, r, &ex, &tok);
    if (ex < 0) continue;
    expert_ptrs wp = expert_at(dm, c->w, ex);
    float sh = 1.0f;
    if (requant) {
      moe_oracle_e4m3_decode_array(c->hq + r * dm->f, dm->f, a);
      sh = c->sh[r];
    } else {
      memcpy(a, c->h + r * dm->f, sizeof(float) * (size_t)dm->f);
    }
    down_row(a, sh, requant, wp.wd, wp.sd, dm->d, dm->f, c->out + r * dm->d);
  }
  free(a);
}

int moe_oracle_expert_down(const oracle_dims *dims, int32_t capacity, const uint8_t *hq,
                           const float *sh, const float *h, const int32_t *sorted_pairs,
                           const int32_t *expert_offsets, const oracle_weights *w, float *y,
                           int nthreads) {
  if (check_dims(dims, w) || !sorted_pairs || !expert_offsets || !y) return 1;
  if (dims->flags & ORACLE_F_NO_REQUANT) {
    if (!h) return 1;
  } else if (!hq || !sh) {
    return 1;
  }
  if ((int64_t)capacity < moe_oracle_capacity(dims->T, dims->E, dims->k_max, dims->block_m))
    return 2;
  stage_ctx c = {dims, capacity, NULL, NULL, hq, sh, h, sorted_pairs, expert_offsets, w, y};
  int64_t rows = (int64_t)capacity + (int64_t)dims->n_shared * dims->T;
  parallel_for(rows, 1, nthreads, down_range, &c);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* step 8: weighted combine back into token order                            */
/* ------------------------------------------------------------------------ */

/* "Routage MoE entre GPU", the last step: the selected experts' outputs are
 * multiplied by their routing weights, summed, and restored to the original
 * token order.  out[t] = 0; out[t] += w[t,j] * y[inv[t,j]] for valid slots j
 * in ascending order; then out[t] += y_shared(s, t) for s ascending (shared
 * experts: weight 1, outside the softmax). */
int moe_oracle_combine(const oracle_dims *dims, int32_t capacity, const float *y,
                       const int32_t *topk_ids, const float *topk_w, const int32_t *inv_pairs,
                       float *out) {
  if (!dims || !y || !topk_ids || !topk_w || !inv_pairs || !out) return 1;
  int32_t d = dims->d, K = dims->k_max;
  for (int64_t t = 0; t < dims->T; ++t) {
    float *o = out + t * d;
    for (int32_t c = 0; c < d; ++c) o[c] = 0.0f;
    for (int32_t j = 0; j < K; ++j) {
      int64_t p = t * K + j;
      if (topk_ids[p] < 0) continue;
      const float *yr = y + (int64_t)inv_pairs[p] * d;
      float wj = topk_w[p];
      for (int32_t c = 0; c < d; ++c) o[c] += wj * yr[c];
    }
    for (int32_t s = 0; s < dims->n_shared; ++s) {
      const float *yr = y + ((int64_t)capacity + (int64_t)s * dims->T + t) * d;
      for (int32_t c = 0; c < d; ++c) o[c] += yr[c];
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* the whole layer, token by token                                           */
/* ------------------------------------------------------------------------ */

typedef struct {
  const oracle_dims *dm;
  const oracle_weights *w;
  const uint8_t *xq;
  const float *sx;
  const int32_t *ids;
  int32_t slots; /* k_max + n_shared rows per token */
  float *y;      /* [T][slots][d] */
} fwd_ctx;

/* Work item i = (token t, slot j): j < k_max is the j-th routed pick (skipped
 * when invalid), j >= k_max is shared expert j - k_max. */
static void forward_range(void *p, int64_t b, int64_t e) {
  fwd_ctx *c = (fwd_ctx *)p;
  const oracle_dims *dm = c->dm;
  int requant = !(dm->flags & ORACLE_F_NO_REQUANT);
  float *xv = (float *)malloc(sizeof(float) * (size_t)dm->d);
  float *h = (float *)malloc(sizeof(float) * (size_t)dm->f);
  float *a = (float *)malloc(sizeof(float) * (size_t)dm->f);
  uint8_t *hq = (uint8_t *)malloc((size_t)dm->f);
  for (int64_t i = b; i < e; ++i) {
    int64_t t = i / c->slots;
    int32_t j = (int32_t)(i % c->slots);
    int32_t ex;
    if (j < dm->k_max) {
      ex = c->ids[t * dm->k_max + j];
      if (ex < 0) continue;
    } else {
      ex = dm->E + (j - dm->k_max);
    }
    expert_ptrs wp = expert_at(dm, c->w, ex);
    moe_oracle_e4m3_decode_array(c->xq + t * dm->d, dm->d, xv);
    gate_up_row(xv, c->sx[t], wp.wg, wp.wu, wp.sg, wp.su, dm->d, dm->f, h);
    float sh = 1.0f;
    if (requant) {
      quantize_row(h, dm->f, hq, &sh);
      moe_oracle_e4m3_decode_array(hq, dm->f, a);
    } else {
      memcpy(a, h, sizeof(float) * (size_t)dm->f);
    }
    down_row(a, sh, requant, wp.wd, wp.sd, dm->d, dm->f, c->y + i * dm->d);
  }
  free(xv);
  free(h);
  free(a);
  free(hq);
}

int moe_oracle_forward(const oracle_dims *dims, const float *x, const float *w_router,
                       const float *router_bias, const int32_t *k_per_token,
                       const oracle_weights *w, const float *logits_override, float *out,
                       int32_t *topk_ids_out, float *topk_w_out, int nthreads) {
  if (check_dims(dims, w) || !x || !out) return 1;
  if (!logits_override && !w_router) return 1;
  const oracle_dims *dm = dims;
  int64_t T = dm->T;
  int rc = 0;
  uint8_t *xq = (uint8_t *)malloc((size_t)(T * dm->d) + 1);
  float *sx = (float *)malloc(sizeof(float) * (size_t)T + 4);
  float *logits = (float *)malloc(sizeof(float) * (size_t)(T * dm->E) + 4);
  int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T * dm->k_max) + 4);
  float *wt = (float *)malloc(sizeof(float) * (size_t)(T * dm->k_max) + 4);
  int32_t slots = dm->k_max + dm->n_shared;
  float *y = (float *)malloc(sizeof(float) * (size_t)(T * slots * dm->d) + 4);
  if (!xq || !sx || !logits || !ids || !wt || !y) {
    rc = 4;
    goto done;
  }
  if ((rc = moe_oracle_quantize_rows(x, (int32_t)T, dm->d, xq, sx)) != 0) goto done;
  if (logits_override)
    memcpy(logits, logits_override, sizeof(float) * (size_t)(T * dm->E));
  else if ((rc = moe_oracle_router_logits(x, w_router, router_bias, (int32_t)T, dm->d, dm->E,
                                           logits, nthreads)) != 0)
    goto done;
  if ((rc = moe_oracle_route_topk(logits, (int32_t)T, dm->E, dm->k_max, k_per_token, ids, wt)) !=
      0)
    goto done;
  {
    fwd_ctx c = {dm, w, xq, sx, ids, slots, y};
    parallel_for(T * slots, 1, nthreads, forward_range, &c);
  }
  for (int64_t t = 0; t < T; ++t) {
    float *o = out + t * dm->d;
    for (int32_t c = 0; c < dm->d; ++c) o[c] = 0.0f;
    for (int32_t j = 0; j < dm->k_max; ++j) {
      if (ids[t * dm->k_max + j] < 0) continue;
      const float *yr = y + (t * slots + j) * dm->d;
      float wj = wt[t * dm->k_max + j];
      for (int32_t c = 0; c < dm->d; ++c) o[c] += wj * yr[c];
    }
    for (int32_t s = 0; s < dm->n_shared; ++s) {
      const float *yr = y + (t * slots + dm->k_max + s) * dm->d;
      for (int32_t c = 0; c < dm->d; ++c) o[c] += yr[c];
    }
  }
  if (topk_ids_out) memcpy(topk_ids_out, ids, sizeof(int32_t) * (size_t)(T * dm->k_max));
  if (topk_w_out) memcpy(topk_w_out, wt, sizeof(float) * (size_t)(T * dm->k_max));
done:
  free(xq);
  free(sx);
  free(logits);
  free(ids);
  free(wt);
  free(y);
  return rc;
}
