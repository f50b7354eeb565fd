/*
 * fp8moe.h -- C ABI of the MI355X (gfx950) W8A8 FP8 Mixture-of-Experts layer.
 *
 * The layer, stated in the blog post "Routage MoE entre GPU": a router reads
 * each token's hidden state and scores every expert, keeps the best k and
 * gives each pick a routing weight; only the picked experts (each a
 * feed-forward network with its own weights) process the token; their
 * outputs are multiplied by the routing weights, summed, and put back in the
 * original token order.  Weights and activations are 8-bit FP8 (W8A8; the
 * Alpha-MoE article, opening section), and the article's section
 * "Comment fonctionne le megakernel" names the stages fused here: routing,
 * gating, expert compute and output combine.
 *
 * Readings taken where the pages are silent (each is a fixed convention of
 * this library):
 *   - FP8 is OCP E4M3FN (bias 7, largest finite 448, no infinities),
 *     round to nearest, ties to even, saturating to +-448.
 *   - Activations: one fp32 scale per token row, s = amax/448; the codes are
 *     e4m3(x * fl(448/amax)); an all-zero row uses s = 1.
 *   - Weights: one fp32 scale per output channel (per row of W_gate, W_up
 *     [f][d] over d; per row of W_down [d][f] over f).
 *   - Router: fp32 logits on the unquantised x, plus an optional bias.
 *   - Top-k: experts ordered by (logit descending, index ascending), -0 and
 *     +0 equal; weights are the softmax over the k selected logits.
 *   - Expert: h = SiLU(g) * u with g, u the dequantised gate/up products;
 *     h is requantised to e4m3 with one scale per (token, expert) row unless
 *     MOE_F_NO_REQUANT is set; y = down projection of h.
 *   - Combine: out[t] = sum_j w[t,j] * y(t, ids[t,j]) + sum_s y_shared(s,t);
 *     shared experts have weight 1 and sit outside the softmax.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns
 *     every buffer; the library keeps no pointer after returning, never
 *     allocates, frees or synchronises.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; device-side faults surface at the
 *     caller's next synchronisation.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failing call returns a non-zero moe_status, enqueues nothing, and
 *     moe_last_error() describes the failure (thread-local text).
 *   - Preconditions the release library does not report: inputs are finite,
 *     every k_per_token[t] is in [1, k_max], every topk_ids entry is -1 or in
 *     [0, E).  Out-of-range values stay memory-safe (a k is clamped to
 *     [1, k_max], an id outside [-1, E) is dropped), but the results are then
 *     undefined.  The debug build of the same sources, libfp8moe_debug.so
 *     (FP8MOE_DEBUG; moe_debug_checks() returns 1), checks them on the
 *     device together with the permutation's index invariants and the GEMM
 *     tiles' channel alignment, waits for its work at the end of every call
 *     that enqueues any, and returns MOE_ERR_DEVICE_CHECK naming the checks
 *     that failed.  It synchronises, so it is not for graph capture or
 *     timing.
 *   - Calls on one stream are ordered; calls on different streams that share
 *     output or workspace buffers race.
 */
#ifndef FP8MOE_H
#define FP8MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8MOE_ABI_VERSION 6

typedef int32_t moe_status;
enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is out of the supported range */
  MOE_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned */
  MOE_ERR_UNSUPPORTED = 4, /* a flag or configuration this build does not run */
  MOE_ERR_WORKSPACE = 5,   /* workspace missing or smaller than moe_workspace_bytes */
  MOE_ERR_HIP = 6,         /* the HIP runtime reported an error at launch */
  MOE_ERR_DEVICE_CHECK = 7 /* debug build only: a device-side check failed */
};

enum {
  MOE_F_NO_REQUANT = 1u << 0, /* keep SiLU*up in fp32 and run the down projection on fp32
                                 products; an accuracy mode, not a fast path */
  MOE_F_PERSISTENT = 1u << 1, /* run the whole layer as one resident-grid (cooperative)
                                 launch, the stages separated by grid-wide barriers inside
                                 the kernel (the fused persistent kernel of the Alpha-MoE
                                 article, section "Comment fonctionne le megakernel"); a
                                 one-wave kernel zeroing the barrier state precedes it.
                                 Routing (ids, weights) is identical to the per-stage path;
                                 outputs agree to rounding.  The workspace then starts with
                                 the barrier state, and the int32 at byte offset 0 of the
                                 workspace is a status word the caller may read after
                                 synchronising: 0 = ok, 1 = a grid barrier timed out (every
                                 wait is bounded, so a grid that cannot run co-resident ends
                                 with this status instead of hanging; outputs are then
                                 invalid).  MOE_ERR_UNSUPPORTED when the device cannot keep
                                 one workgroup resident per compute unit */
  MOE_F_FUSED_COMBINE = 1u << 2 /* reserved for a combine fused into the down projection's
                                 epilogue.  Not built: with expert-major tiles the only fusion
                                 is a floating-point accumulation of each token's slots in
                                 arrival order, which is neither in slot order nor
                                 reproducible run to run; the weighted sum here is taken in
                                 slot order by its own kernel.  Every call that takes dims
                                 returns MOE_ERR_UNSUPPORTED when it is set */
};

/* Limits checked by every call. */
#define MOE_MAX_EXPERTS 512
#define MOE_MAX_K 32
#define MOE_MAX_HIDDEN 16384 /* d: the router keeps a token's row in 64 KB of LDS */
#define MOE_MAX_FFN 16384    /* f: requantisation keeps an h row in registers */

typedef struct {
  int32_t T;        /* tokens, >= 1 */
  int32_t d;        /* hidden size, multiple of 64, at most MOE_MAX_HIDDEN */
  int32_t f;        /* expert intermediate size, multiple of 64, at most MOE_MAX_FFN */
  int32_t E;        /* routed experts, 1..512 */
  int32_t k_max;    /* slots per token, 1..min(E, 32) */
  int32_t n_shared; /* always-on shared experts, >= 0 */
  int32_t block_m;  /* expert segments padded to a multiple of this: 1, 16, 32, 64 or 128 */
  uint32_t flags;   /* MOE_F_* */
} moe_dims;

/* Expert weights: e4m3 codes (one byte each) in MFMA tile order, and fp32
 * per-output-channel scales.
 *
 * The tile order is part of the boundary on purpose: the grouped GEMMs
 * stream every active expert's weights from HBM once per step, and in this
 * order each 16-byte load of a wave belongs to a fully contiguous 1 KB piece
 * (row-major rows would need 16 separate 64-byte half-lines per load).
 * moe_pack_weights converts row-major codes once, at weight-load time.
 *
 * Tile order of a code matrix W [R][C] (R output channels, a multiple of 16;
 * C inputs, a multiple of 64), as written by moe_pack_weights: with
 * CT = ceil(C / 128), 2048-byte tiles indexed by (r / 16) * CT + c / 128, and
 * inside a tile, for l = (r % 16) + 16 * ((c % 64) / 16):
 *   W[r][c] at byte  l * 16 + c % 16          when c % 128 <  64,
 *              byte  1024 + l * 16 + c % 16   when c % 128 >= 64;
 * bytes for c >= C are zero.  A tile is the weight operand of one
 * v_mfma_f32_16x16x128_f8f6f4 (lane l reads 16 contiguous bytes from each
 * half), so a wave loads it as two fully contiguous 1 KB pieces.
 * Size of one matrix: moe_packed_weight_bytes(R, C) = R * CT * 128. */
typedef struct {
  const uint8_t *w_gate, *w_up; /* [E] tile-order matrices of [f][d] */
  const float *s_gate, *s_up;   /* [E][f] */
  const uint8_t *w_down;        /* [E] tile-order matrices of [d][f] */
  const float *s_down;          /* [E][d] */
  const uint8_t *ws_gate, *ws_up, *ws_down; /* shared experts: same layouts with */
  const float *ss_gate, *ss_up, *ss_down;   /* n_shared in place of E; NULL when 0 */
} moe_weights;

/* ------------------------------------------------------------------------ */
/* Single steps                                                              */
/* ------------------------------------------------------------------------ */

/* Per-row e4m3 quantisation (the W8A8 activation / weight encoding).
 * x [rows][cols] fp32 -> q [rows][cols] e4m3 codes, scale [rows] fp32 with
 * x ~= dec(q) * scale.  Used for per-token activations and, on weight
 * matrices, for per-output-channel weight scales.
 * cols: multiple of 4; x 16-byte aligned; q 4-byte aligned. */
moe_status moe_quantize_rows(const float *x, int32_t rows, int32_t cols, uint8_t *q, float *scale,
                             void *stream);

/* Bytes of one weight matrix of R output channels by C inputs in tile order
 * (see moe_weights); 0 when R is not a positive multiple of 16 or C not a
 * positive multiple of 64. */
int64_t moe_packed_weight_bytes(int32_t rows, int32_t cols);

/* Reorders row-major e4m3 codes [rows][cols] into tile order (moe_weights)
 * at packed (moe_packed_weight_bytes(rows, cols) bytes, zero padding
 * included).  rows multiple of 16, cols multiple of 64 up to 16384; codes
 * and packed 16-byte aligned and not overlapping. */
moe_status moe_pack_weights(const uint8_t *codes, int32_t rows, int32_t cols, uint8_t *packed,
                            void *stream);

/* Router scores ("Routage MoE entre GPU", the router paragraph):
 * logits[t][e] = sum_i x[t][i] * w_router[e][i] (+ bias[e]), fp32.
 * x [T][d], w_router [E][d], bias [E] or NULL, logits [T][E]. */
moe_status moe_router_logits(const float *x, const float *w_router, const float *bias, int32_t T,
                             int32_t d, int32_t E, float *logits, void *stream);

/* Top-k selection with routing weights (same paragraph: the router keeps the
 * best experts and emits one weight per pick).  For token t with
 * k_t = k_per_token ? k_per_token[t] : k_max: topk_ids[t][0..k_t) are the
 * first k_t experts in (logit desc, index asc) order and topk_w the softmax of
 * their logits; slots k_t..k_max-1 get id -1 and weight 0.
 * logits [T][E], k_per_token [T] or NULL, topk_ids/topk_w [T][k_max]. */
moe_status moe_route_topk(const float *logits, int32_t T, int32_t E, int32_t k_max,
                          const int32_t *k_per_token, int32_t *topk_ids, float *topk_w,
                          void *stream);

/* Rows a permutation needs: T*k_max + E*(block_m-1). */
int64_t moe_capacity(int32_t T, int32_t E, int32_t k_max, int32_t block_m);

/* Dispatch on one device (the activation movement of "Routage MoE entre GPU"
 * becomes a grouping of (token, slot) pairs by expert; the inverse map is
 * what restores token order at the end).  Pair p = t*k_max + j is valid when
 * topk_ids[p] >= 0.  Expert e's segment starts at
 * expert_offsets[e] = sum_{e'<e} ceil(cnt[e']/block_m)*block_m and holds its
 * pairs in ascending p, then the sentinel T*k_max; rows past the last segment
 * also hold the sentinel.  block_expert[b] is the expert owning rows
 * [b*block_m, (b+1)*block_m), -1 past the last segment.  inv_pairs[p] is p's
 * row, -1 for an invalid pair.  n_blocks[0] = expert_offsets[E] / block_m.
 * Deterministic: the result is unique.
 * sorted_pairs [capacity], expert_offsets [E+1], block_expert
 * [ceil(capacity/block_m)], inv_pairs [T*k_max], n_blocks [1]. */
moe_status moe_permute(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k_max,
                       int32_t block_m, int32_t capacity, int32_t *sorted_pairs,
                       int32_t *expert_offsets, int32_t *block_expert, int32_t *inv_pairs,
                       int32_t *n_blocks, void *stream);

/* The same permutation with a device workspace for the per-slice expert
 * counts of large batches (T*k_max >= 4096 pairs, cut into slices of 1024):
 * with it the permutation takes two launches instead of three; the outputs
 * are those of moe_permute bit for bit.  moe_permute_workspace_bytes gives
 * the size (0 when the batch needs none: then workspace may be NULL); the
 * workspace must be 16-byte aligned, caller-owned, and not touched by
 * anything else while the work is in flight.  MOE_ERR_WORKSPACE when it is
 * missing or too small; other errors as moe_permute.  moe_fused_forward runs
 * this form on its own workspace. */
size_t moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t k_max);
moe_status moe_permute_ws(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k_max,
                          int32_t block_m, int32_t capacity, int32_t *sorted_pairs,
                          int32_t *expert_offsets, int32_t *block_expert, int32_t *inv_pairs,
                          int32_t *n_blocks, void *workspace, size_t workspace_bytes,
                          void *stream);

/* "Expert rows" layout used by the three expert stages below: rows
 * [0, capacity) follow sorted_pairs (padding rows hold garbage or zeros);
 * row capacity + s*T + t is token t for shared expert s.
 * rows_total = capacity + n_shared*T.  w_gate[e][o][i] below is the logical
 * element (row o, column i) of expert e's matrix, stored in tile order. */

/* Gate/up grouped GEMM with the SwiGLU epilogue, for every expert row:
 *   g[o] = (sum_i dec(xq[t][i]) * dec(w_gate[e][o][i])) * sx[t] * s_gate[e][o]
 *   u[o] likewise with w_up;  h[row][o] = SiLU(g[o]) * u[o]   (fp32)
 * dims->flags is ignored.  xq [T][d], sx [T], h [rows_total][f]. */
moe_status moe_expert_gate_up(const moe_dims *dims /*host*/, int32_t capacity, const uint8_t *xq,
                              const float *sx, const int32_t *sorted_pairs,
                              const int32_t *expert_offsets, const moe_weights *w /*host*/,
                              float *h, void *stream);

/* Down-projection grouped GEMM for every expert row:
 *   y[row][c] = (sum_o dec(hq[row][o]) * dec(w_down[e][c][o])) * sh[row] * s_down[e][c]
 * hq [rows_total][f] e4m3, sh [rows_total], y [rows_total][d] fp32.
 * With MOE_F_NO_REQUANT in dims->flags the input is instead h [rows_total][f]
 * fp32 (hq, sh ignored, may be NULL):
 *   y[row][c] = (sum_o h[row][o] * dec(w_down[e][c][o])) * s_down[e][c]. */
moe_status moe_expert_down(const moe_dims *dims /*host*/, int32_t capacity, const uint8_t *hq,
                           const float *sh, const float *h, const int32_t *sorted_pairs,
                           const int32_t *expert_offsets, const moe_weights *w /*host*/, float *y,
                           void *stream);

/* Weighted combine back into token order ("Routage MoE entre GPU", the last
 * step):  out[t] = sum over valid j ascending of topk_w[t][j] * y[inv_pairs[t*k_max+j]]
 *                  + sum over s ascending of y[capacity + s*T + t].
 * y [rows_total][d], out [T][d]. */
moe_status moe_combine(const moe_dims *dims /*host*/, int32_t capacity, const float *y,
                       const int32_t *topk_ids, const float *topk_w, const int32_t *inv_pairs,
                       float *out, void *stream);

/* ------------------------------------------------------------------------ */
/* The whole layer                                                           */
/* ------------------------------------------------------------------------ */

/* Bytes of device workspace moe_fused_forward needs for these dims. */
size_t moe_workspace_bytes(const moe_dims *dims /*host*/);

/* Forward pass of one W8A8 FP8 MoE layer: quantise x, router logits (or
 * logits_override), top-k + weights, permutation, gate/up + SiLU*up,
 * requantisation, down projection, weighted combine.  Intermediates stay in
 * the workspace: h in fp32, hq in e4m3, and the down projection's outputs y
 * in fp16 on their way to the combine (values beyond +-65504 saturate; with
 * MOE_F_NO_REQUANT, h and y stay fp32).  Where one workgroup spans all of f
 * (f <= 192) the requantisation is done in the gate/up epilogue and h never
 * reaches memory; hq and its scales are the same bit for bit.
 * x [T][d] fp32; w_router [E][d] (may be NULL when logits_override is given);
 * router_bias [E] or NULL; k_per_token [T] or NULL (all k_max);
 * logits_override [T][E] or NULL; out [T][d] fp32;
 * topk_ids_out / topk_w_out [T][k_max] or NULL;
 * workspace: device buffer of at least moe_workspace_bytes(dims), 256-byte
 * aligned, not touched by anything else while the work is in flight. */
moe_status moe_fused_forward(const moe_dims *dims /*host*/, const float *x, const float *w_router,
                             const float *router_bias, const int32_t *k_per_token,
                             const moe_weights *w /*host*/, const float *logits_override,
                             float *out, int32_t *topk_ids_out, float *topk_w_out,
                             void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * forward pass as moe_fused_forward, with the workspace taken from a device
 * array inside the library instead of a caller buffer.  The array,
 * MOE_STATIC_WORKSPACE_BYTES, exists once per GPU the library runs on and
 * is held until the process ends; its device address is looked up on the
 * first call on each device.  The call allocates nothing (no hipMalloc, no
 * allocating library routine); the caller still passes the inputs and
 * outputs.  Dims whose workspace (moe_workspace_bytes) exceeds the array
 * return MOE_ERR_WORKSPACE with nothing enqueued -- the decode-sized layers
 * fit, prefill-sized ones need moe_fused_forward.  Nothing in the array has
 * to start at zero (every stage writes what the next one reads).  Every call
 * on one GPU shares that GPU's array: calls whose work overlaps on one GPU
 * (other streams, other threads) race; serialise them.  Other arguments and
 * errors as moe_fused_forward. */
#define MOE_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)
moe_status moe_fused_forward_noalloc(const moe_dims *dims /*host*/, const float *x,
                                     const float *w_router, const float *router_bias,
                                     const int32_t *k_per_token, const moe_weights *w /*host*/,
                                     const float *logits_override, float *out,
                                     int32_t *topk_ids_out, float *topk_w_out, void *stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                               */
/* ------------------------------------------------------------------------ */

/* Decode batching by expert affinity ("ELDR : Microsoft et KAIST accélèrent
 * le décodage des MoE": a decode step loads the weights of every distinct
 * expert its batch activates; changing only which tokens share a batch
 * changes no token's output).  Orders a pool of n tokens, given their
 * routing, into batches of `batch` tokens (the last one shorter when n is
 * not a multiple) that activate few distinct experts: each batch starts
 * from the lowest-numbered unplaced token, then repeatedly takes the
 * unplaced token that adds the fewest experts not yet in the batch (ties:
 * the lowest number).  Deterministic.  HOST memory: ids [n][k] (-1 = empty
 * slot, else in [0, E); a repeated id counts once), order [n] out, a
 * permutation of 0..n-1 -- batch b is order[b*batch .. min(n, (b+1)*batch)).
 * Synchronous, no device work, no allocation visible to the caller.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (also for an id outside [-1, E)). */
moe_status moe_group_tokens(const int32_t *ids /*host*/, int32_t n, int32_t k, int32_t E,
                            int32_t batch, int32_t *order /*host*/);

/* Quality-tier batching by routing budget ("MoE-Prism: Disentangling
 * Monolithic Experts …", section Méthodologie B, offline throughput-oriented
 * mode: requests sorted by their k and grouped into tiers; a tier's residual
 * batch is dispatched at once or merged into the next tier, which serves it at
 * the larger k).  Plans the dispatch of a pool of n tokens with routing
 * budgets k_per_token into batches of at most `batch` tokens, each run at one
 * k: tiers in ascending k, tokens of a tier in ascending number, full batches
 * cut from the front of the tier's pool.  A residual of r < batch tokens of
 * tier k is merged into the next tier when r * k_next < overhead + r * k
 * (`overhead`: the cost of one more batch, in (token, slot) pairs), otherwise
 * dispatched as a short batch; a merged residual leads the next tier's pool,
 * and the last tier's residual is always dispatched.  No token is served
 * below its budget.  Deterministic.  HOST memory: k_per_token [n], each in
 * [1, MOE_MAX_K]; out: order [n] (tokens in dispatch order), batch_start
 * [n+1] (batch b is order[batch_start[b] .. batch_start[b+1])), batch_k [n]
 * (the k batch b runs at), n_batches [1].  Synchronous, no device work.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (n < 0, batch < 1, overhead < 0, a
 * budget outside [1, MOE_MAX_K]). */
moe_status moe_k_tiers(const int32_t *k_per_token /*host*/, int32_t n, int32_t batch,
                       int32_t overhead, int32_t *order /*host*/, int32_t *batch_start /*host*/,
                       int32_t *batch_k /*host*/, int32_t *n_batches /*host*/);

/* ------------------------------------------------------------------------ */

/* Stage timing (instrumentation, not part of the layer): moe_fused_forward
 * that also records stage_events[i] on its stream just before stage i
 * (0 quantise + router logits, 1 top-k, 2 permutation, 3 gate/up,
 * 4 requantisation, 5 down, 6 combine) and stage_events[7] after the last
 * one; a stage fused into the one before it (top-k into routing, the
 * requantisation into gate/up) has its two events back to back.  stage_events: host array of n_events >= MOE_N_STAGE_EVENTS hipEvent_t
 * handles created and owned by the caller, or NULL (then identical to
 * moe_fused_forward).  The library records the events during this call only
 * and keeps nothing.  Returns MOE_ERR_SHAPE when stage_events is given with
 * n_events < MOE_N_STAGE_EVENTS; other errors as moe_fused_forward. */
#define MOE_N_STAGE_EVENTS 8
moe_status moe_fused_forward_timed(const moe_dims *dims /*host*/, const float *x,
                                   const float *w_router, const float *router_bias,
                                   const int32_t *k_per_token, const moe_weights *w /*host*/,
                                   const float *logits_override, float *out,
                                   int32_t *topk_ids_out, float *topk_w_out, void *workspace,
                                   size_t workspace_bytes, void *const *stage_events /*host*/,
                                   int32_t n_events, void *stream);

const char *moe_status_str(moe_status s);
const char *moe_last_error(void); /* thread-local detail of this thread's last failing call */
int32_t moe_abi_version(void);
/* 1 in the debug build (device-side checks, see the conventions above), 0 in
 * the release library. */
int32_t moe_debug_checks(void);

#ifdef __cplusplus
}
#endif
#endif /* FP8MOE_H */
