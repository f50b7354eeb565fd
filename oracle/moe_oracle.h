/*
 * moe_oracle.h -- CPU oracle for the W8A8 FP8 Mixture-of-Experts layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or helper with the GPU library.
 *
 * The layer (router / top-k / weighted sum: the blog post "Routage MoE entre
 * GPU"; W8A8 FP8 and the fused stage list: the Alpha-MoE article, opening
 * section and "Comment fonctionne le megakernel"):
 *
 *   xq, sx   = per-token e4m3 quantisation of x                 (quantize_rows)
 *   logits   = x . W_r^T + b   (fp32, on the unquantised x)     (router_logits)
 *   ids, w   = first k_t experts in (logit desc, index asc) order,
 *              softmax over those k_t logits                    (route_topk)
 *   per selected (token, expert) row:
 *     g, u   = dequantised fp8 products, h = SiLU(g) * u        (expert_gate_up)
 *     hq, sh = per-row e4m3 requantisation of h (unless disabled)
 *     y      = dequantised fp8 down projection                  (expert_down)
 *   out[t]   = sum_j w[t,j] * y(t, ids[t,j]) + sum_s y_shared(s, t)   (combine)
 *
 * All floating point is IEEE fp32 with a fixed order (ascending reduction
 * index) and is compiled with -ffp-contract=off.  e4m3 is OCP E4M3FN: bias 7,
 * 3 mantissa bits, largest finite value 448, no infinities, NaN = S.1111.111.
 *
 * Row layout shared by the stage functions ("expert rows"): rows
 * [0, capacity) hold the routed (token, slot) pairs in the padded,
 * expert-sorted order written by moe_oracle_permute; rows
 * capacity + s*T + t hold token t for shared expert s.
 *
 * Buffers are host memory owned by the caller.  Functions returning int give
 * 0 on success and a positive code on an argument error (nothing written).
 * nthreads <= 0 means "every CPU this process may run on".
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_F_NO_REQUANT 1u /* keep the SiLU*up intermediate in fp32 */

typedef struct {
  int32_t T;        /* tokens */
  int32_t d;        /* hidden size */
  int32_t f;        /* expert FFN intermediate size */
  int32_t E;        /* routed experts */
  int32_t k_max;    /* slots per token (columns of ids / w) */
  int32_t n_shared; /* always-on shared experts (weight 1, outside the softmax) */
  int32_t block_m;  /* expert segments are padded to a multiple of this */
  uint32_t flags;   /* ORACLE_F_* */
} oracle_dims;

typedef struct {
  const uint8_t *w_gate, *w_up; /* [E][f][d] e4m3 codes */
  const float *s_gate, *s_up;   /* [E][f]    per-output-channel scales */
  const uint8_t *w_down;        /* [E][d][f] */
  const float *s_down;          /* [E][d] */
  const uint8_t *ws_gate, *ws_up, *ws_down; /* shared experts: same layouts with */
  const float *ss_gate, *ss_up, *ss_down;   /* n_shared in place of E (NULL if 0) */
} oracle_weights;

/* ---- e4m3 codec ---------------------------------------------------------- */
uint8_t moe_oracle_e4m3_encode(float v); /* nearest, ties to even code; |v| >= 448 -> +-448 */
float moe_oracle_e4m3_decode(uint8_t c); /* exact value of a code (NaN for 0x7F / 0xFF) */
void moe_oracle_e4m3_encode_array(const float *v, int64_t n, uint8_t *out);
void moe_oracle_e4m3_decode_array(const uint8_t *c, int64_t n, float *out);
/* Checks the bit encoder against a nearest-value search over the finite codes
 * for every fp32 bit pattern in [lo, hi).  Returns the mismatch count;
 * *first_bad receives the first mismatching pattern. */
int64_t moe_oracle_codec_selfcheck(uint64_t lo, uint64_t hi, uint32_t *first_bad, int nthreads);

/* ---- layer steps ---------------------------------------------------------- */
int64_t moe_oracle_capacity(int32_t T, int32_t E, int32_t k_max, int32_t block_m);

int moe_oracle_quantize_rows(const float *x, int32_t rows, int32_t cols, uint8_t *q, float *scale);

int moe_oracle_router_logits(const float *x, const float *w_router, const float *bias, int32_t T,
                             int32_t d, int32_t E, float *logits, int nthreads);

int moe_oracle_route_topk(const float *logits, int32_t T, int32_t E, int32_t k_max,
                          const int32_t *k_per_token, int32_t *topk_ids, float *topk_w);

int moe_oracle_permute(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k_max,
                       int32_t block_m, int32_t capacity, int32_t *sorted_pairs,
                       int32_t *expert_offsets, int32_t *block_expert, int32_t *inv_pairs,
                       int32_t *n_blocks);

/* h[row][f] for every real expert row (padding rows are left untouched). */
int moe_oracle_expert_gate_up(const oracle_dims *dims, int32_t capacity, const uint8_t *xq,
                              const float *sx, const int32_t *sorted_pairs,
                              const int32_t *expert_offsets, const oracle_weights *w, float *h,
                              int nthreads);

/* y[row][d]: from hq/sh (requantised) or, with ORACLE_F_NO_REQUANT, from h. */
int moe_oracle_expert_down(const oracle_dims *dims, int32_t capacity, const uint8_t *hq,
                           const float *sh, const float *h, const int32_t *sorted_pairs,
                           const int32_t *expert_offsets, const oracle_weights *w, float *y,
                           int nthreads);

int moe_oracle_combine(const oracle_dims *dims, int32_t capacity, const float *y,
                       const int32_t *topk_ids, const float *topk_w, const int32_t *inv_pairs,
                       float *out);

/* The whole layer, computed token by token straight from the definition
 * (no permutation).  logits_override (nullable) replaces the router output. */
int moe_oracle_forward(const oracle_dims *dims, const float *x, const float *w_router,
                       const float *router_bias, const int32_t *k_per_token,
                       const oracle_weights *w, const float *logits_override, float *out,
                       int32_t *topk_ids_out, float *topk_w_out, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
