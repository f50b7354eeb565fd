// abi.hip -- the C ABI (include/fp8moe.h): host-side validation, workspace
// layout, tile-shape choice and kernel enqueueing.  No allocation, no
// synchronisation, no state kept between calls except the thread-local error
// text and each device's compute-unit count.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/fp8moe.h"
#include "internal.hpp"

using namespace fp8moe;

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

moe_status ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

}  // namespace

// The error text of the calling thread, for host-side entry points defined
// in other files.
namespace fp8moe {
moe_status fail_status(moe_status code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}
moe_status ok_status() { return ok(); }
}  // namespace fp8moe

namespace {

// The end of an entry point that enqueued work: in the debug build, wait for
// it and report the device checks that failed; in the release library only
// the status.
moe_status done(moe_status s, const char *fn) {
  if (s) return s;
#ifdef FP8MOE_DEBUG
  const uint32_t b = debug_take_route() | debug_take_permute() | debug_take_expert() |
                     debug_take_persistent();
  if (b)
    return fail(MOE_ERR_DEVICE_CHECK, "%s: device checks failed (0x%x):%s%s%s%s%s%s%s", fn, b,
                (b & 1u) ? " k_per_token outside [1, k_max];" : "",
                (b & 2u) ? " non-finite logit or activation row;" : "",
                (b & 4u) ? " top-k id outside [-1, E);" : "",
                (b & 8u) ? " work item outside its expert's rows;" : "",
                (b & 16u) ? " row index outside the row space;" : "",
                (b & 32u) ? " GEMM tile channel not a multiple of 16;" : "",
                (b & 0x80000000u) ? " the check words could not be read;" : "");
#endif
  return ok();
}

moe_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

bool block_m_ok(int32_t bm) { return bm == 1 || bm == 16 || bm == 32 || bm == 64 || bm == 128; }

moe_status check_dims(const moe_dims *d, const char *fn) {
  if (!d) return fail(MOE_ERR_NULL, "%s: dims is NULL", fn);
  if (d->T < 1) return fail(MOE_ERR_SHAPE, "%s: T=%d must be >= 1", fn, d->T);
  if (d->d < 64 || d->d % 64 || d->d > MOE_MAX_HIDDEN)
    return fail(MOE_ERR_SHAPE, "%s: d=%d must be a multiple of 64 in [64, %d]", fn, d->d, MOE_MAX_HIDDEN);
  if (d->f < 64 || d->f % 64 || d->f > MOE_MAX_FFN)
    return fail(MOE_ERR_SHAPE, "%s: f=%d must be a multiple of 64 in [64, %d]", fn, d->f, MOE_MAX_FFN);
  if (d->E < 1 || d->E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_SHAPE, "%s: E=%d must be in [1, %d]", fn, d->E, MOE_MAX_EXPERTS);
  if (d->k_max < 1 || d->k_max > d->E || d->k_max > MOE_MAX_K)
    return fail(MOE_ERR_SHAPE, "%s: k_max=%d must be in [1, min(E, %d)]", fn, d->k_max, MOE_MAX_K);
  if (d->n_shared < 0) return fail(MOE_ERR_SHAPE, "%s: n_shared=%d must be >= 0", fn, d->n_shared);
  if (!block_m_ok(d->block_m))
    return fail(MOE_ERR_SHAPE, "%s: block_m=%d must be 1, 16, 32, 64 or 128", fn, d->block_m);
  if (d->flags & MOE_F_FUSED_COMBINE)
    return fail(MOE_ERR_UNSUPPORTED,
                "%s: MOE_F_FUSED_COMBINE is not built (the combine runs in slot order in its own "
                "kernel)", fn);
  if (d->flags & ~(uint32_t)(MOE_F_NO_REQUANT | MOE_F_PERSISTENT))
    return fail(MOE_ERR_UNSUPPORTED, "%s: unknown flags 0x%x", fn, d->flags);
  // all row indices must fit in int32
  const int64_t rows = (int64_t)d->T * d->k_max + (int64_t)d->E * (d->block_m - 1) +
                       (int64_t)d->n_shared * d->T;
  if (rows * (int64_t)(d->d > d->f ? d->d : d->f) > ((int64_t)1 << 40) || rows >= ((int64_t)1 << 31))
    return fail(MOE_ERR_SHAPE, "%s: layer too large (%lld expert rows)", fn, (long long)rows);
  return MOE_OK;
}

moe_status check_weights(const moe_dims *d, const moe_weights *w, const char *fn) {
  if (!w) return fail(MOE_ERR_NULL, "%s: weights is NULL", fn);
  if (!w->w_gate || !w->w_up || !w->w_down || !w->s_gate || !w->s_up || !w->s_down)
    return fail(MOE_ERR_NULL, "%s: a routed expert weight or scale pointer is NULL", fn);
  if (d->n_shared > 0 &&
      (!w->ws_gate || !w->ws_up || !w->ws_down || !w->ss_gate || !w->ss_up || !w->ss_down))
    return fail(MOE_ERR_NULL, "%s: n_shared=%d but a shared expert pointer is NULL", fn, d->n_shared);
  const void *p16[] = {w->w_gate, w->w_up, w->w_down, w->ws_gate, w->ws_up, w->ws_down};
  for (const void *p : p16)
    if (p && !aligned(p, 16)) return fail(MOE_ERR_ALIGN, "%s: weight codes must be 16-byte aligned", fn);
  const void *p4[] = {w->s_gate, w->s_up, w->s_down, w->ss_gate, w->ss_up, w->ss_down};
  for (const void *p : p4)
    if (p && !aligned(p, 4)) return fail(MOE_ERR_ALIGN, "%s: scales must be 4-byte aligned", fn);
  return MOE_OK;
}

ExpertWeights to_internal(const moe_weights *w) {
  return ExpertWeights{w->w_gate,  w->w_up,  w->w_down,  w->s_gate,  w->s_up,  w->s_down,
                       w->ws_gate, w->ws_up, w->ws_down, w->ss_gate, w->ss_up, w->ss_down};
}

int64_t capacity_of(int32_t T, int32_t E, int32_t k, int32_t bm) {
  return (int64_t)T * k + (int64_t)E * (bm - 1);
}

// Row-pass size for the grouped GEMMs: 16*msub rows per pass, sized so that a
// decode-sized batch keeps all of an expert's rows in one pass (its weights
// then stream from HBM once).  mean + 4 sigma of a binomial expert load, in
// units of 16 rows, rounded up to a power of two, at most 8.
int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return (v && *v) ? atoi(v) : dflt;
}

int32_t choose_msub(const moe_dims *d) {
  // tile-tuning override (power of two, 1..8)
  const int forced = env_int("FP8MOE_MSUB", 0);
  if (forced == 1 || forced == 2 || forced == 4 || forced == 8 || forced == 16) return forced;
  const double mean = (double)d->T * d->k_max / d->E;
  const double est = mean + 4.0 * sqrt(mean) + 2.0;
  int32_t m = 1;
  while (m < 16 && 16.0 * m < est) m <<= 1;
  return m;
}

// Experts expected to receive at least one token (uniform routing).
double expected_active(const moe_dims *d) {
  const double E = d->E;
  return E * (1.0 - pow(1.0 - (double)d->k_max / E, (double)d->T));
}

// Row-pass height for work items that outgrow 16*msub rows.  A token picks
// an expert at most once, so routing can send up to the whole batch to one
// expert; items are cut at 16*msub_big rows, msub_big covering the batch
// where it can (at most 8).  Equal to msub where one shape serves (or the
// row pass is forced).
int32_t choose_msub_big(const moe_dims *d, int32_t msub) {
  if (msub >= 8) return msub;
  const int forced = env_int("FP8MOE_MSUB_BIG", 0);  // tile-tuning override
  if (forced == 2 || forced == 4 || forced == 8) return forced > msub ? forced : msub;
  if (env_int("FP8MOE_MSUB", 0) > 0) return msub;
  const int64_t most = ((int64_t)d->T + d->block_m - 1) / d->block_m * d->block_m;
  int32_t m = msub;
  while (m < 8 && 16 * (int64_t)m < most) m <<= 1;
  return m;
}

// Non-temporal weight loads pay off where each weight byte is read by one
// workgroup (every expert's rows, routed and shared, expected in one work
// item); weights re-read by several items lose.  The K range itself does not
// matter: with the hint on the short-K down projections as well (an earlier
// rule asked for K >= 2048 bytes) the MoE-Prism-shaped layer (K = 192, the
// A-resident tile) went 261 -> 246 us and the Qwen3-shaped T=64 layer at 16
// distinct experts (K = 768) 53.2 -> 51.5 us; Qwen3 T=64 at ~127 experts and
// DeepSeek T=32 (K = 1408) stayed within 1 %.
bool stream_weights(const moe_dims *d, int32_t msub_big) {
  const int forced = env_int("FP8MOE_NT", -1);  // tile-tuning override
  if (forced == 0 || forced == 1) return forced == 1;
  const double mean = (double)d->T * d->k_max / d->E;
  const double est = mean + 4.0 * sqrt(mean) + 2.0;
  const int64_t chunk = 16 * (int64_t)msub_big;
  return est <= chunk && (d->n_shared == 0 || d->T <= chunk);
}

// Expected work items of the grouped GEMMs (rows cut into 16*msub chunks).
double expected_items(const moe_dims *d, int32_t msub) {
  const double chunk = 16.0 * msub;
  const double mean = (double)d->T * d->k_max / d->E;
  const double rows = ceil(mean / d->block_m) * d->block_m;  // padded segment
  const double per = rows > chunk ? ceil(rows / chunk) : 1.0;
  return expected_active(d) * per + d->n_shared * ceil(d->T / chunk);
}

// Grouped-GEMM geometry.  A workgroup of W compute waves, each holding nb
// weight operands of 16 rows (2 or 4), covers W * ch_wave output channels
// of one work item and one K split.  With nb 2, up to five compute waves
// and row passes of up to 64 rows, the model lets two workgroups share a CU,
// otherwise one.  A simple model picks (W, nb, splits): workgroups run in whole rounds
// of resident ones; a CU streams weights at a rate that grows with the
// weight loads it keeps in flight (resident waves * nb) up to about six
// two-operand waves; a workgroup's time is proportional to its weight
// bytes; each K split adds one fp32 slab of y to write and to read back.
// The estimated time per CU,
//   rounds * wg_per_cu * W*ch_wave*K/splits / min(1, waves_per_cu*nb/12)
//   + splits * 2 * rows * N * 4 / CUs,
// is minimised, ties going to the larger W and the fewer splits.
struct GemmPlan {
  int32_t waves, splits, nb;
};

// Compute units of the current device, queried once per device ordinal
// (256 on MI355X; the planner's rounds depend on it).
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    cus = 256;
  if (dev < kMaxDevices) g_cus[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

GemmPlan plan_gemm(const moe_dims *d, int32_t msub, bool gate_up) {
  const int kCUs = device_cus();
  const double items = expected_items(d, msub);
  const int N = gate_up ? d->f : d->d;
  const int K = gate_up ? d->d : d->f;
  const double rows = (double)d->T * d->k_max + (double)d->n_shared * d->T;
  const int forced_dn = gate_up ? 0 : env_int("FP8MOE_DOWN_WAVES", 0);  // tile-tuning overrides
  const int forced = forced_dn > 0 ? forced_dn : env_int("FP8MOE_WAVES", 0);
  const int forced_nb = env_int("FP8MOE_NB", 0);
  const int forced_splits = env_int("FP8MOE_DOWN_SPLITS", 0);
  const bool can_split = !gate_up && !(d->flags & MOE_F_NO_REQUANT);
  GemmPlan best{4, 1, 2};
  double best_t = 1e300;
  // four operands per wave measured no faster than two on this chip's
  // decode and prefill shapes; they stay a tile-tuning option
  const int nb_first = (forced_nb == 4 && msub <= 8) ? 4 : 2;
  for (int nb = nb_first; nb >= 2; nb -= 2) {
    const int ch_wave = gate_up ? 8 * nb : 16 * nb;
    // 256-row passes: the prefill kernel's eight waves, or a forced wave
    // count on the loader-wave kernel (at most six computing waves)
    const int maxw = msub > 8 ? (forced >= 1 ? kGemmMaxWaves16 : kPfWaves)
                              : nb > 2 ? kGemmMaxThreadsWide / 64 - 1 : kGemmMaxWaves;
    for (int W = maxw; W >= 1; --W) {
      if (forced >= 1 && forced <= maxw && W != forced) continue;
      if (msub > 8 && forced < 1 && W != kPfWaves) continue;
      // Two workgroups per CU only for passes of up to 64 rows: with 128-row
      // passes one workgroup of more waves streamed faster (DeepSeek-shaped
      // T=512 down projection, 5 waves x 2 -> 7 waves x 1: 72 -> 63 us;
      // MoE-Prism-shaped gate/up 3 x 2 -> 6 x 1: 82 -> 80 us).
      const int per_cu = (nb == 2 && W <= 5 && msub <= 4) ? 2 : 1;
      const double slots = (double)kCUs * per_cu;
      const int tiles = (N + W * ch_wave - 1) / (W * ch_wave);
      const double rate = std::min(1.0, W * per_cu * nb / 12.0);
      int last = 0;
      for (int want = 1; want <= (can_split ? kMaxDownSplits : 1); ++want) {
        const int req = forced_splits > 0 ? std::min(forced_splits, kMaxDownSplits) : want;
        const int sp = can_split ? down_splits_used(d->f, msub, req) : 1;
        if (sp == last) continue;
        last = sp;
        const double n = items * tiles * sp;
        const double rounds = ceil(n / slots);
        const double t = rounds * per_cu * (double)W * ch_wave * K / sp / rate +
                         sp * 2.0 * rows * N * 4.0 / kCUs;
        // gate/up ties go to the smaller wave count (more workgroups, so
        // more of them overlap one another's start and end; W is tried
        // downwards): Qwen3-shaped T=64, W=8 and W=6 tie, 79 -> 73 us with
        // W=6.  The down projection keeps the first of equals (its ties
        // went the wrong way: Mixtral-shaped T=256 down 90 -> 120 us).
        if (gate_up ? t <= best_t * (1.0 + 1e-9) : t < best_t * (1.0 - 1e-9)) {
          best_t = t;
          best = GemmPlan{W, sp, nb};
        }
      }
    }
  }
  return best;
}

// Workspace layout of moe_fused_forward (all pieces 256-byte aligned).
struct Layout {
  size_t bar, xq, sx, logits, ids, w, sorted, offsets, block_expert, inv, n_blocks, items, n_items, h,
      hq, sh, y, pcnt, total;
  int32_t capacity, rows_total, max_items, row_chunk, msub, msub_big, splits;
  bool nt_gu, nt_dn;  // non-temporal weight loads
  GemmPlan gu, dn;
  bool ares_gu, ares_dn;     // A-resident tiles (short K)
  bool rq_gu;                // gate/up with the requantisation fused in (f <= 16*kRqMaxWaves)
  int32_t ntg_gu, ntg_dn;    // their N-tiles per workgroup
};

// A-resident tiles for a short-K GEMM: the items' whole K range in LDS
// (ares_fits), two-operand plans of up to 128-row items, outside the single
// persistent launch.  FP8MOE_ARES=0 keeps the per-tile kernels (tile tuning).
bool use_ares(const moe_dims *d, const GemmPlan &p, int32_t msub_big, bool gate_up) {
  static const int env = env_int("FP8MOE_ARES", 1);
  if (!env || (d->flags & MOE_F_PERSISTENT) || p.nb != 2 || msub_big > 8) return false;
  if (!gate_up && (d->flags & MOE_F_NO_REQUANT)) return false;
  return ares_fits(msub_big, gate_up ? d->d : d->f);
}

// Waves of an A-resident workgroup: the plan's waves plus the loader's slot
// (every wave computes), at most kAresMaxWaves.
int32_t ares_waves(const GemmPlan &p) { return std::min(p.waves + 1, kAresMaxWaves); }

// N-tiles per A-resident workgroup: about two workgroups per slot in all.
int32_t ares_ntg(const moe_dims *d, const GemmPlan &p, int32_t msub_big, bool gate_up) {
  const int N = gate_up ? d->f : d->d;
  const int ch_wg = ares_waves(p) * (gate_up ? 16 : 32);
  const int n_tiles = (N + ch_wg - 1) / ch_wg;
  const double units = expected_items(d, msub_big) * n_tiles;
  const double slots = (double)device_cus() * (ares_waves(p) <= 6 ? 2 : 1);
  const int forced = env_int("FP8MOE_ARES_NTG", 0);  // tile-tuning override
  int ntg = forced > 0 ? forced : (int)(units / (2.0 * slots));
  // the workgroup's weight scales are staged in LDS (32 floats per wave and tile)
  ntg = std::min(ntg, kAresScaleFloats / (ares_waves(p) * 32));
  return std::max(1, std::min(ntg, n_tiles));
}

size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }

Layout layout_of(const moe_dims *d) {
  Layout L{};
  L.capacity = (int32_t)capacity_of(d->T, d->E, d->k_max, d->block_m);
  L.rows_total = L.capacity + d->n_shared * d->T;
  L.msub = choose_msub(d);
  L.gu = plan_gemm(d, L.msub, true);
  L.dn = plan_gemm(d, L.msub, false);
  const bool persistent = d->flags & MOE_F_PERSISTENT;
  // the single launch runs one row-pass shape: items cut at 16*msub rows
  L.msub_big = (L.gu.nb == 2 && L.dn.nb == 2 && !persistent) ? choose_msub_big(d, L.msub) : L.msub;
  L.row_chunk = 16 * L.msub_big;
  // A-resident tiles where a workgroup gets at least two tiles of short K
  L.ntg_gu = ares_ntg(d, L.gu, L.msub_big, true);
  L.ntg_dn = ares_ntg(d, L.dn, L.msub_big, false);
  L.ares_gu = use_ares(d, L.gu, L.msub_big, true) && L.ntg_gu >= 2;
  L.ares_dn = use_ares(d, L.dn, L.msub_big, false) && L.ntg_dn >= 2;
  L.splits = L.ares_dn ? 1 : L.dn.splits;
  // Where one workgroup of up to twelve two-operand waves spans all of f, the
  // gate/up epilogue requantises h itself (no fp32 h, no requantisation
  // launch), in row passes of at most 64 rows over the same work items (cut
  // at 16*msub_big rows).  FP8MOE_RQ=0 keeps the separate requantisation.
  L.rq_gu = !(d->flags & (MOE_F_NO_REQUANT | MOE_F_PERSISTENT)) && !L.ares_gu &&
            L.msub_big <= 8 && d->f <= 16 * kRqMaxWaves && env_int("FP8MOE_RQ", 1) != 0;
  if (L.rq_gu) L.gu = GemmPlan{(d->f + 15) / 16, 1, 2};
  L.nt_gu = (L.gu.nb == 2 || L.rq_gu) && L.msub <= 8 && stream_weights(d, L.msub_big);
  L.nt_dn = L.dn.nb == 2 && L.msub <= 8 && !(d->flags & MOE_F_NO_REQUANT) &&
            stream_weights(d, L.msub_big);
  L.max_items = max_work_items(d->T, d->E, d->k_max, d->block_m, d->n_shared, L.row_chunk);
  const size_t T = d->T, P = (size_t)d->T * d->k_max, R = L.rows_total;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = up256(o + bytes);
    return at;
  };
  L.bar = persistent ? take(kPersistBarBytes) : 0;  // first: the status word at offset 0
  L.xq = take(T * d->d);
  L.sx = take(T * 4);
  L.logits = take(T * d->E * 4);
  L.ids = take(P * 4);
  L.w = take(P * 4);
  L.sorted = take((size_t)L.capacity * 4);
  L.offsets = take((size_t)(d->E + 1) * 4);
  L.block_expert = take((size_t)((L.capacity + d->block_m - 1) / d->block_m) * 4);
  L.inv = take(P * 4);
  L.n_blocks = take(4);
  L.items = take((size_t)L.max_items * sizeof(WorkItem));
  L.n_items = take(4);
  L.h = take(R * d->f * 4);
  L.hq = take(R * d->f);
  L.sh = take(R * 4);
  // the fused path keeps y in fp16 (fp32 in the no-requant accuracy mode)
  L.y = take((size_t)L.splits * R * d->d * ((d->flags & MOE_F_NO_REQUANT) ? 4 : 2));
  L.pcnt = take((size_t)permute_counts_ints(d->T, d->E, d->k_max) * 4);  // slice counts
  L.total = o;
  return L;
}

RowSpace row_space(const moe_dims *d, int32_t capacity, const int32_t *sorted_pairs,
                          const int32_t *expert_offsets) {
  RowSpace rs{};
  rs.T = d->T;
  rs.d = d->d;
  rs.f = d->f;
  rs.E = d->E;
  rs.S = d->n_shared;
  rs.k_max = d->k_max;
  rs.capacity = capacity;
  rs.sorted_pairs = sorted_pairs;
  rs.expert_offsets = expert_offsets;
  return rs;
}

// Host-side checks of moe_fused_forward's arguments (everything but the
// workspace).
moe_status check_forward(const moe_dims *dims, const float *x, const float *w_router,
                         const moe_weights *w, const float *logits_override, const float *out,
                         const char *fn) {
  moe_status s = check_dims(dims, fn);
  if (s) return s;
  if ((s = check_weights(dims, w, fn))) return s;
  if (!x || !out) return fail(MOE_ERR_NULL, "%s: x and out are required", fn);
  if (!w_router && !logits_override)
    return fail(MOE_ERR_NULL, "%s: w_router is required unless logits_override is given", fn);
  if (!aligned(x, 16) || !aligned(out, 16) || (w_router && !aligned(w_router, 16)))
    return fail(MOE_ERR_ALIGN, "%s: x, out and w_router must be 16-byte aligned", fn);
  return MOE_OK;
}

// Enqueues the whole layer on `st` with workspace `ws` laid out as L;
// ev: NULL, or MOE_N_STAGE_EVENTS events recorded around the stages.
moe_status enqueue_forward(const moe_dims *dims, const float *x, const float *w_router,
                           const float *router_bias, const int32_t *k_per_token,
                           const moe_weights *w, const float *logits_override, float *out,
                           int32_t *topk_ids_out, float *topk_w_out, char *ws, const Layout &L,
                           hipEvent_t const *ev, hipStream_t st) {
  moe_status s = MOE_OK;
  uint8_t *xq = reinterpret_cast<uint8_t *>(ws + L.xq);
  float *sx = reinterpret_cast<float *>(ws + L.sx);
  float *logits = reinterpret_cast<float *>(ws + L.logits);
  int32_t *ids = topk_ids_out ? topk_ids_out : reinterpret_cast<int32_t *>(ws + L.ids);
  float *tw = topk_w_out ? topk_w_out : reinterpret_cast<float *>(ws + L.w);
  int32_t *sorted = reinterpret_cast<int32_t *>(ws + L.sorted);
  int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
  int32_t *block_expert = reinterpret_cast<int32_t *>(ws + L.block_expert);
  int32_t *inv = reinterpret_cast<int32_t *>(ws + L.inv);
  int32_t *n_blocks = reinterpret_cast<int32_t *>(ws + L.n_blocks);
  WorkItem *items = reinterpret_cast<WorkItem *>(ws + L.items);
  int32_t *n_items = reinterpret_cast<int32_t *>(ws + L.n_items);
  float *h = reinterpret_cast<float *>(ws + L.h);
  uint8_t *hq = reinterpret_cast<uint8_t *>(ws + L.hq);
  float *sh = reinterpret_cast<float *>(ws + L.sh);
  float *y = reinterpret_cast<float *>(ws + L.y);
  const bool requant = !(dims->flags & MOE_F_NO_REQUANT);
  _Float16 *y16 = requant ? reinterpret_cast<_Float16 *>(ws + L.y) : nullptr;
  auto mark = [&](int i) {
    if (ev) (void)hipEventRecord(ev[i], st);
  };

  if (dims->flags & MOE_F_PERSISTENT) {
    if (L.gu.nb != 2 || L.dn.nb != 2)
      return fail(MOE_ERR_UNSUPPORTED,
                  "moe_fused_forward: MOE_F_PERSISTENT runs two-operand GEMM tiles only");
    const int32_t grid = persistent_grid(L.msub, device_cus());
    if (grid < 1)
      return fail(MOE_ERR_UNSUPPORTED,
                  "moe_fused_forward: the single-launch kernel cannot keep one workgroup "
                  "resident on every compute unit of this device");
    PersistentLaunch p{};
    p.rs = row_space(dims, L.capacity, sorted, offsets);
    p.rs.items = items;
    p.rs.n_items = n_items;
    p.rs.max_items = L.max_items;
    p.w = to_internal(w);
    p.x = x;
    p.w_router = w_router;
    p.bias = router_bias;
    p.kpt = k_per_token;
    p.logits_override = logits_override;
    p.logits = logits;
    p.xq = xq;
    p.sx = sx;
    p.ids = ids;
    p.tw = tw;
    p.sorted = sorted;
    p.offsets = offsets;
    p.block_expert = block_expert;
    p.inv = inv;
    p.n_blocks = n_blocks;
    p.items = items;
    p.n_items = n_items;
    p.h = h;
    p.hq = hq;
    p.sh = sh;
    p.y = y;
    p.y16 = y16;
    p.out = out;
    p.bar = reinterpret_cast<uint32_t *>(ws + L.bar);
    p.block_m = dims->block_m;
    p.row_chunk = L.row_chunk;
    p.msub = L.msub;
    p.splits = requant ? L.splits : 1;
    p.no_requant = !requant;
    mark(0);
    if ((s = hip_status(launch_persistent(p, grid, st), "persistent"))) return s;
    for (int i = 1; i < MOE_N_STAGE_EVENTS; ++i) mark(i);
    return ok();
  }

  mark(0);
  const float *lg = logits_override;
  if (!lg && route_fused_applies(dims->T, dims->E)) {
    // one launch: logits, quantised x, top-k
    if ((s = hip_status(launch_route_topk_fused(x, w_router, router_bias, dims->T, dims->d,
                                                dims->E, dims->k_max, k_per_token, logits, xq, sx,
                                                ids, tw, st),
                        "route")))
      return s;
    mark(1);
  } else if (!lg && route_tile_applies(dims->T, dims->E)) {
    if ((s = hip_status(launch_route_prefill(x, w_router, router_bias, dims->T, dims->d, dims->E,
                                             dims->k_max, k_per_token, logits, xq, sx, ids, tw, st),
                        "route")))
      return s;
    mark(1);
  } else {
    if (!lg) {
      if ((s = hip_status(launch_route_logits(x, w_router, router_bias, dims->T, dims->d, dims->E,
                                              logits, xq, sx, st),
                          "router")))
        return s;
      lg = logits;
    } else if ((s = hip_status(launch_quantize_rows(x, dims->T, dims->d, xq, sx, st), "quantize"))) {
      return s;
    }
    mark(1);
    if ((s = hip_status(launch_topk(lg, dims->T, dims->E, dims->k_max, k_per_token, ids, tw, st),
                        "topk")))
      return s;
  }
  mark(2);
  if ((s = hip_status(launch_permute(ids, dims->T, dims->E, dims->k_max, dims->block_m, L.capacity,
                                     sorted, offsets, block_expert, inv, n_blocks, items, n_items,
                                     L.row_chunk, dims->n_shared, st,
                                     reinterpret_cast<int32_t *>(ws + L.pcnt)),
                      "permute")))
    return s;
  RowSpace rs = row_space(dims, L.capacity, sorted, offsets);
  rs.items = items;
  rs.n_items = n_items;
  rs.max_items = L.max_items;
  const ExpertWeights ew = to_internal(w);
  mark(3);
  if (L.ares_gu) {
    if ((s = hip_status(launch_ares(rs, xq, sx, ew, h, nullptr, true, L.msub_big, ares_waves(L.gu),
                                    L.ntg_gu, L.nt_gu, st),
                        "gate_up")))
      return s;
  } else if (L.rq_gu) {
    if ((s = hip_status(launch_gate_up_rq(rs, xq, sx, ew, hq, sh, L.msub, L.gu.waves, L.nt_gu, st),
                        "gate_up")))
      return s;
  } else if ((s = hip_status(launch_gate_up(rs, xq, sx, ew, h, L.msub, L.msub_big, L.gu.waves, L.gu.nb, L.nt_gu, st), "gate_up"))) {
    return s;
  }
  mark(4);
  if (requant) {
    if (!L.rq_gu && (s = hip_status(launch_requant(rs, h, hq, sh, st), "requant"))) return s;
    mark(5);
    if (L.ares_dn) {
      if ((s = hip_status(launch_ares(rs, hq, sh, ew, nullptr, y16, false, L.msub_big,
                                      ares_waves(L.dn), L.ntg_dn, L.nt_dn, st),
                          "down")))
        return s;
    } else if ((s = hip_status(launch_down(rs, hq, sh, nullptr, ew, nullptr, y16, L.msub, L.msub_big, L.splits, L.dn.waves, L.dn.nb, L.nt_dn, st),
                               "down"))) {
      return s;
    }
  } else {
    mark(5);
    if ((s = hip_status(launch_down(rs, nullptr, nullptr, h, ew, y, nullptr, L.msub, L.msub, 1, L.dn.waves, L.dn.nb, false, st), "down")))
      return s;
  }
  mark(6);
  if ((s = hip_status(launch_combine(rs, y, y16, L.splits, ids, tw, inv, out, st), "combine"))) return s;
  mark(7);
  return ok();
}

// Allocation-free entry point: the workspace lives in this file-scope device
// array (one copy per GPU, held until the process ends).  Its device
// address is taken once per device with hipGetSymbolAddress and kept; host
// code never passes the array's own name to a kernel.
}  // namespace

// At most MOE_STATIC_WORKSPACE_BYTES; see the header.  File scope, internal
// linkage: in host code `scratch` names a host-side stand-in, never passed to
// a kernel or a copy -- only the address hipGetSymbolAddress returns is.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_WORKSPACE_BYTES];

namespace {

constexpr size_t kStaticScratchBytes = MOE_STATIC_WORKSPACE_BYTES;

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

moe_status scratch_of_current_device(void **ptr, const char *fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MOE_ERR_UNSUPPORTED, "%s: device ordinal %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOE_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

const char *moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "unsupported shape";
    case MOE_ERR_ALIGN: return "misaligned pointer";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_DEVICE_CHECK: return "device check failed (debug build)";
    default: return "unknown status";
  }
}

const char *moe_last_error(void) { return g_err; }

int32_t moe_abi_version(void) { return FP8MOE_ABI_VERSION; }

int32_t moe_debug_checks(void) {
#ifdef FP8MOE_DEBUG
  return 1;
#else
  return 0;
#endif
}

int64_t moe_capacity(int32_t T, int32_t E, int32_t k_max, int32_t block_m) {
  return capacity_of(T, E, k_max, block_m);
}

moe_status moe_quantize_rows(const float *x, int32_t rows, int32_t cols, uint8_t *q, float *scale,
                             void *stream) {
  const char *fn = "moe_quantize_rows";
  if (!x || !q || !scale) return fail(MOE_ERR_NULL, "%s: x, q and scale are required", fn);
  if (rows < 0 || cols < 4 || cols % 4)
    return fail(MOE_ERR_SHAPE, "%s: rows=%d, cols=%d (cols must be a positive multiple of 4)", fn,
                rows, cols);
  if (!aligned(x, 16) || !aligned(q, 4) || !aligned(scale, 4))
    return fail(MOE_ERR_ALIGN, "%s: x must be 16-byte and q 4-byte aligned", fn);
  moe_status s = hip_status(launch_quantize_rows(x, rows, cols, q, scale, as_stream(stream)), fn);
  return done(s, fn);
}

int64_t moe_packed_weight_bytes(int32_t rows, int32_t cols) {
  if (rows <= 0 || rows % 16 || cols <= 0 || cols % 64) return 0;
  return (int64_t)rows * ((cols + 127) / 128) * 128;
}

moe_status moe_pack_weights(const uint8_t *codes, int32_t rows, int32_t cols, uint8_t *packed,
                            void *stream) {
  const char *fn = "moe_pack_weights";
  if (!codes || !packed) return fail(MOE_ERR_NULL, "%s: codes and packed are required", fn);
  if (moe_packed_weight_bytes(rows, cols) == 0 || cols > MOE_MAX_FFN)
    return fail(MOE_ERR_SHAPE, "%s: rows=%d cols=%d (rows a multiple of 16, cols of 64 up to %d)",
                fn, rows, cols, MOE_MAX_FFN);
  if (!aligned(codes, 16) || !aligned(packed, 16))
    return fail(MOE_ERR_ALIGN, "%s: codes and packed must be 16-byte aligned", fn);
  const uintptr_t a = (uintptr_t)codes, b = (uintptr_t)packed;
  const uintptr_t na = (uintptr_t)rows * cols, nb = (uintptr_t)moe_packed_weight_bytes(rows, cols);
  if (a < b + nb && b < a + na) return fail(MOE_ERR_SHAPE, "%s: codes and packed overlap", fn);
  moe_status s = hip_status(launch_pack_weights(codes, rows, cols, packed, as_stream(stream)), fn);
  return done(s, fn);
}

moe_status moe_router_logits(const float *x, const float *w_router, const float *bias, int32_t T,
                             int32_t d, int32_t E, float *logits, void *stream) {
  const char *fn = "moe_router_logits";
  if (!x || !w_router || !logits) return fail(MOE_ERR_NULL, "%s: x, w_router and logits are required", fn);
  if (T < 0 || d < 64 || d % 64 || d > MOE_MAX_HIDDEN || E < 1 || E > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_SHAPE, "%s: T=%d d=%d E=%d (d multiple of 64 up to %d, E in [1,%d])", fn,
                T, d, E, MOE_MAX_HIDDEN, MOE_MAX_EXPERTS);
  if (!aligned(x, 16) || !aligned(w_router, 16))
    return fail(MOE_ERR_ALIGN, "%s: x and w_router must be 16-byte aligned", fn);
  moe_status s =
      hip_status(launch_router(x, w_router, bias, T, d, E, logits, as_stream(stream)), fn);
  return done(s, fn);
}

moe_status moe_route_topk(const float *logits, int32_t T, int32_t E, int32_t k_max,
                          const int32_t *k_per_token, int32_t *topk_ids, float *topk_w,
                          void *stream) {
  const char *fn = "moe_route_topk";
  if (!logits || !topk_ids || !topk_w) return fail(MOE_ERR_NULL, "%s: logits, topk_ids and topk_w are required", fn);
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k_max < 1 || k_max > E || k_max > MOE_MAX_K)
    return fail(MOE_ERR_SHAPE, "%s: T=%d E=%d k_max=%d", fn, T, E, k_max);
  moe_status s = hip_status(
      launch_topk(logits, T, E, k_max, k_per_token, topk_ids, topk_w, as_stream(stream)), fn);
  return done(s, fn);
}

static moe_status permute_checked(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k_max,
                                  int32_t block_m, int32_t capacity, int32_t *sorted_pairs,
                                  int32_t *expert_offsets, int32_t *block_expert,
                                  int32_t *inv_pairs, int32_t *n_blocks, int32_t *counts,
                                  void *stream, const char *fn) {
  if (!topk_ids || !sorted_pairs || !expert_offsets || !block_expert || !inv_pairs || !n_blocks)
    return fail(MOE_ERR_NULL, "%s: every array is required", fn);
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k_max < 1 || k_max > MOE_MAX_K ||
      !block_m_ok(block_m) || (int64_t)T * k_max >= ((int64_t)1 << 30))
    return fail(MOE_ERR_SHAPE, "%s: T=%d E=%d k_max=%d block_m=%d", fn, T, E, k_max, block_m);
  if ((int64_t)capacity < capacity_of(T, E, k_max, block_m))
    return fail(MOE_ERR_SHAPE, "%s: capacity=%d < T*k_max + E*(block_m-1) = %lld", fn, capacity,
                (long long)capacity_of(T, E, k_max, block_m));
  moe_status s = hip_status(launch_permute(topk_ids, T, E, k_max, block_m, capacity, sorted_pairs,
                                           expert_offsets, block_expert, inv_pairs, n_blocks,
                                           nullptr, nullptr, 0, 0, as_stream(stream), counts),
                            fn);
  return done(s, fn);
}

moe_status moe_permute(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k_max,
                       int32_t block_m, int32_t capacity, int32_t *sorted_pairs,
                       int32_t *expert_offsets, int32_t *block_expert, int32_t *inv_pairs,
                       int32_t *n_blocks, void *stream) {
  return permute_checked(topk_ids, T, E, k_max, block_m, capacity, sorted_pairs, expert_offsets,
                         block_expert, inv_pairs, n_blocks, nullptr, stream, "moe_permute");
}

size_t moe_permute_workspace_bytes(int32_t T, int32_t E, int32_t k_max) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || k_max < 1 || k_max > MOE_MAX_K ||
      (int64_t)T * k_max >= ((int64_t)1 << 30))
    return 0;
  return (size_t)permute_counts_ints(T, E, k_max) * 4;
}

moe_status moe_permute_ws(const int32_t *topk_ids, int32_t T, int32_t E, int32_t k_max,
                          int32_t block_m, int32_t capacity, int32_t *sorted_pairs,
                          int32_t *expert_offsets, int32_t *block_expert, int32_t *inv_pairs,
                          int32_t *n_blocks, void *workspace, size_t workspace_bytes,
                          void *stream) {
  const char *fn = "moe_permute_ws";
  const size_t need = moe_permute_workspace_bytes(T, E, k_max);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes < %zu", fn, workspace_bytes, need);
  if (need > 0 && !aligned(workspace, 16))
    return fail(MOE_ERR_ALIGN, "%s: the workspace must be 16-byte aligned", fn);
  return permute_checked(topk_ids, T, E, k_max, block_m, capacity, sorted_pairs, expert_offsets,
                         block_expert, inv_pairs, n_blocks,
                         need > 0 ? static_cast<int32_t *>(workspace) : nullptr, stream, fn);
}


static moe_status check_stage(const moe_dims *dims, int32_t capacity, const moe_weights *w,
                              const int32_t *sorted_pairs, const int32_t *expert_offsets,
                              const char *fn) {
  moe_status s = check_dims(dims, fn);
  if (s) return s;
  if ((s = check_weights(dims, w, fn))) return s;
  if (!sorted_pairs || !expert_offsets)
    return fail(MOE_ERR_NULL, "%s: sorted_pairs and expert_offsets are required", fn);
  const int64_t need = capacity_of(dims->T, dims->E, dims->k_max, dims->block_m);
  if ((int64_t)capacity < need || (int64_t)capacity + (int64_t)dims->n_shared * dims->T >= ((int64_t)1 << 31))
    return fail(MOE_ERR_SHAPE, "%s: capacity=%d must be >= %lld", fn, capacity, (long long)need);
  return MOE_OK;
}

moe_status moe_expert_gate_up(const moe_dims *dims, int32_t capacity, const uint8_t *xq,
                              const float *sx, const int32_t *sorted_pairs,
                              const int32_t *expert_offsets, const moe_weights *w, float *h,
                              void *stream) {
  const char *fn = "moe_expert_gate_up";
  moe_status s = check_stage(dims, capacity, w, sorted_pairs, expert_offsets, fn);
  if (s) return s;
  if (!xq || !sx || !h) return fail(MOE_ERR_NULL, "%s: xq, sx and h are required", fn);
  if (!aligned(xq, 16)) return fail(MOE_ERR_ALIGN, "%s: xq must be 16-byte aligned", fn);
  RowSpace rs = row_space(dims, capacity, sorted_pairs, expert_offsets);
  const int32_t msub = choose_msub(dims);
  const GemmPlan gp = plan_gemm(dims, msub, true);
  const int32_t mbig = gp.nb == 2 ? choose_msub_big(dims, msub) : msub;
  const bool nt = gp.nb == 2 && msub <= 8 && stream_weights(dims, mbig);
  s = hip_status(launch_gate_up(rs, xq, sx, to_internal(w), h, msub, mbig, gp.waves, gp.nb, nt,
                                as_stream(stream)),
                 fn);
  return done(s, fn);
}

moe_status moe_expert_down(const moe_dims *dims, int32_t capacity, const uint8_t *hq,
                           const float *sh, const float *h, const int32_t *sorted_pairs,
                           const int32_t *expert_offsets, const moe_weights *w, float *y,
                           void *stream) {
  const char *fn = "moe_expert_down";
  moe_status s = check_stage(dims, capacity, w, sorted_pairs, expert_offsets, fn);
  if (s) return s;
  const bool f32 = dims->flags & MOE_F_NO_REQUANT;
  if (!y) return fail(MOE_ERR_NULL, "%s: y is required", fn);
  if (f32 ? !h : (!hq || !sh))
    return fail(MOE_ERR_NULL, "%s: %s required", fn, f32 ? "h is" : "hq and sh are");
  if ((f32 && !aligned(h, 16)) || (!f32 && !aligned(hq, 16)))
    return fail(MOE_ERR_ALIGN, "%s: the activation rows must be 16-byte aligned", fn);
  RowSpace rs = row_space(dims, capacity, sorted_pairs, expert_offsets);
  const int32_t msub = choose_msub(dims);
  const GemmPlan dp = plan_gemm(dims, msub, false);
  const int32_t mbig = dp.nb == 2 ? choose_msub_big(dims, msub) : msub;
  const bool nt = !f32 && dp.nb == 2 && msub <= 8 && stream_weights(dims, mbig);
  s = hip_status(launch_down(rs, f32 ? nullptr : hq, sh, f32 ? h : nullptr, to_internal(w), y, nullptr,
                             msub, mbig, 1, dp.waves, dp.nb, nt, as_stream(stream)),
                 fn);
  return done(s, fn);
}

moe_status moe_combine(const moe_dims *dims, int32_t capacity, const float *y,
                       const int32_t *topk_ids, const float *topk_w, const int32_t *inv_pairs,
                       float *out, void *stream) {
  const char *fn = "moe_combine";
  moe_status s = check_dims(dims, fn);
  if (s) return s;
  if (!y || !topk_ids || !topk_w || !inv_pairs || !out)
    return fail(MOE_ERR_NULL, "%s: y, topk_ids, topk_w, inv_pairs and out are required", fn);
  if (!aligned(y, 16) || !aligned(out, 16))
    return fail(MOE_ERR_ALIGN, "%s: y and out must be 16-byte aligned", fn);
  if ((int64_t)capacity < capacity_of(dims->T, dims->E, dims->k_max, dims->block_m))
    return fail(MOE_ERR_SHAPE, "%s: capacity=%d too small", fn, capacity);
  RowSpace rs = row_space(dims, capacity, nullptr, nullptr);
  s = hip_status(launch_combine(rs, y, nullptr, 1, topk_ids, topk_w, inv_pairs, out, as_stream(stream)), fn);
  return done(s, fn);
}

size_t moe_workspace_bytes(const moe_dims *dims) {
  if (check_dims(dims, "moe_workspace_bytes")) return 0;
  return layout_of(dims).total;
}

moe_status moe_fused_forward(const moe_dims *dims, const float *x, const float *w_router,
                             const float *router_bias, const int32_t *k_per_token,
                             const moe_weights *w, const float *logits_override, float *out,
                             int32_t *topk_ids_out, float *topk_w_out, void *workspace,
                             size_t workspace_bytes, void *stream) {
  return moe_fused_forward_timed(dims, x, w_router, router_bias, k_per_token, w, logits_override,
                                 out, topk_ids_out, topk_w_out, workspace, workspace_bytes, nullptr,
                                 0, stream);
}

moe_status moe_fused_forward_timed(const moe_dims *dims, const float *x, const float *w_router,
                                   const float *router_bias, const int32_t *k_per_token,
                                   const moe_weights *w, const float *logits_override, float *out,
                                   int32_t *topk_ids_out, float *topk_w_out, void *workspace,
                                   size_t workspace_bytes, void *const *stage_events,
                                   int32_t n_events, void *stream) {
  const char *fn = "moe_fused_forward";
  moe_status s = check_forward(dims, x, w_router, w, logits_override, out, fn);
  if (s) return s;
  if (stage_events && n_events < MOE_N_STAGE_EVENTS)
    return fail(MOE_ERR_SHAPE, "%s: %d stage events given, %d needed", fn, n_events,
                MOE_N_STAGE_EVENTS);
  const Layout L = layout_of(dims);
  if (!workspace || workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn,
                workspace ? workspace_bytes : (size_t)0, L.total);
  if (!aligned(workspace, 256))
    return fail(MOE_ERR_ALIGN, "%s: workspace must be 256-byte aligned", fn);
  return done(enqueue_forward(dims, x, w_router, router_bias, k_per_token, w, logits_override, out,
                              topk_ids_out, topk_w_out, static_cast<char *>(workspace), L,
                              reinterpret_cast<hipEvent_t const *>(stage_events), as_stream(stream)),
              fn);
}

moe_status moe_fused_forward_noalloc(const moe_dims *dims, const float *x, const float *w_router,
                                     const float *router_bias, const int32_t *k_per_token,
                                     const moe_weights *w, const float *logits_override,
                                     float *out, int32_t *topk_ids_out, float *topk_w_out,
                                     void *stream) {
  const char *fn = "moe_fused_forward_noalloc";
  moe_status s = check_forward(dims, x, w_router, w, logits_override, out, fn);
  if (s) return s;
  const Layout L = layout_of(dims);
  if (L.total > kStaticScratchBytes)
    return fail(MOE_ERR_WORKSPACE,
                "%s: these dims need %zu bytes of workspace, above the %zu-byte static scratch "
                "array; use moe_fused_forward with a caller workspace",
                fn, L.total, kStaticScratchBytes);
  void *ws = nullptr;
  if ((s = scratch_of_current_device(&ws, fn))) return s;
  return done(enqueue_forward(dims, x, w_router, router_bias, k_per_token, w, logits_override, out,
                              topk_ids_out, topk_w_out, static_cast<char *>(ws), L, nullptr,
                              as_stream(stream)),
              fn);
}

}  // extern "C"
