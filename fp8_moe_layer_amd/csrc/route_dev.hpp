// route_dev.hpp -- device functions of the routing steps (router logits,
// top-k + softmax weights), shared by the per-stage kernels and the
// persistent single-launch kernel.
//
// Layer statement: "Routage MoE entre GPU" (router paragraph): the router
// scores every expert from the token's hidden state, keeps the best k and
// emits one routing weight per pick.
#pragma once
#include "common.hpp"

namespace fp8moe {

// ------------------------------------------------------------------ router, decode-sized
// d is cut into parts of kDotPart floats.  A wave sums a part with lanes
// striding it 4 floats at a time (all of a lane's loads issued before its
// FMAs), then a wave-wide sum; the logit is the sum of the part sums in part
// order (+ bias).  So the logit is the same whether one wave walks the parts
// or several waves take one part each.
constexpr int kDotVec = 8;                 // float4 per lane per part
constexpr int kDotPart = kDotVec * 4 * 64; // 2048 floats

// One part starting at `base`: returns its sum (in every lane); x's values
// stay in xv and their absolute maximum is folded into amax.
__device__ __forceinline__ float router_part_wave(const float *__restrict__ xr,
                                                  const float *__restrict__ w, int d, int base,
                                                  int lane, v4f (&xv)[kDotVec], float &amax) {
  v4f wv[kDotVec];
#pragma unroll
  for (int j = 0; j < kDotVec; ++j) {
    const int i = base + (j * 64 + lane) * 4;
    xv[j] = i < d ? *reinterpret_cast<const v4f *>(xr + i) : v4f{0.f, 0.f, 0.f, 0.f};
    wv[j] = i < d ? *reinterpret_cast<const v4f *>(w + i) : v4f{0.f, 0.f, 0.f, 0.f};
  }
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < kDotVec; ++j) {
    acc = fmaf(xv[j].x, wv[j].x, acc);
    acc = fmaf(xv[j].y, wv[j].y, acc);
    acc = fmaf(xv[j].z, wv[j].z, acc);
    acc = fmaf(xv[j].w, wv[j].w, acc);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(xv[j].x), fabsf(xv[j].y)),
                             fmaxf(fabsf(xv[j].z), fabsf(xv[j].w))));
  }
  return wave_sum(acc);
}

// e4m3 codes of x's values in xv (one part), given the row's amax.
__device__ __forceinline__ void quantize_part_wave(const v4f (&xv)[kDotVec], int d, int base,
                                                   float amax, uint8_t *__restrict__ q, int lane) {
  const float r = amax != 0.0f ? kE4m3Max / amax : 1.0f;
#pragma unroll
  for (int j = 0; j < kDotVec; ++j) {
    const int i = base + (j * 64 + lane) * 4;
    if (i < d) *reinterpret_cast<uint32_t *>(q + i) = e4m3x4(xv[j].x * r, xv[j].y * r, xv[j].z * r, xv[j].w * r);
  }
}

// The (token t, expert e) logit by one wave walking the parts; the wave of
// expert 0 also quantises its token's row (re-reading it past one part).
// Returns the logit in every lane.
__device__ __forceinline__ float router_dot_wave(const float *__restrict__ x,
                                                 const float *__restrict__ wr,
                                                 const float *__restrict__ bias, int d, int E,
                                                 float *__restrict__ logits,
                                                 uint8_t *__restrict__ xq, float *__restrict__ sx,
                                                 int t, int e, int lane) {
  const float *xr = x + (size_t)t * d;
  const float *w = wr + (size_t)e * d;
  float logit = 0.0f, amax = 0.0f;
  v4f xv[kDotVec];
  for (int base = 0; base < d; base += kDotPart) {
    const float ps = router_part_wave(xr, w, d, base, lane, xv, amax);
    logit = base == 0 ? ps : logit + ps;
  }
  if (bias) logit += bias[e];
  if (lane == 0) logits[(size_t)t * E + e] = logit;
  if (e == 0 && xq) {
    amax = wave_max(amax);
    uint8_t *q = xq + (size_t)t * d;
    if (d <= kDotPart) {
      quantize_part_wave(xv, d, 0, amax, q, lane);
    } else {
      const float r = amax != 0.0f ? kE4m3Max / amax : 1.0f;
      for (int i = lane * 4; i < d; i += kWave * 4) {
        const v4f v = *reinterpret_cast<const v4f *>(xr + i);
        *reinterpret_cast<uint32_t *>(q + i) = e4m3x4(v.x * r, v.y * r, v.z * r, v.w * r);
      }
    }
    if (lane == 0) sx[t] = amax != 0.0f ? amax / kE4m3Max : 1.0f;
  }
  return logit;
}

// ------------------------------------------------------------------ router, tiled
// Batches with many (token, expert) pairs: logits = X . W_r^T as an fp32
// GEMM on v_mfma_f32_16x16x4_f32.  One call computes the 32 tokens x 64
// experts tile at (t0, e0); K advances 64 floats at a time through LDS (rows
// padded to 68 floats so the per-lane reads hit distinct banks), the next
// chunk's global loads in flight while the current one is multiplied.
// Threads 0..255 compute (wave w owns tokens [16*(w&1), +16) x experts
// [32*(w>>1), +32)); any further threads of the workgroup only join the
// barriers.  xs, ws: LDS of kRT*kRS and kRE*kRS floats.
constexpr int kRT = 32, kRE = 64, kRK = 64, kRS = kRK + 4;
constexpr int kRouterTileLdsFloats = (kRT + kRE) * kRS;

__device__ __forceinline__ void router_tile(const float *__restrict__ x,
                                            const float *__restrict__ wr,
                                            const float *__restrict__ bias, int T, int d, int E,
                                            float *__restrict__ logits, int t0, int e0, float *xs,
                                            float *ws) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool active = tid < 256;
  const int th = wave & 1, eh = wave >> 1;
  const int lr = lane & 15, lk = lane >> 4;
  v4f acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  // the next K chunk is fetched into registers while the current one is used
  constexpr int XJ = kRT * kRK / 4 / 256, WJ = kRE * kRK / 4 / 256;
  v4f xr[XJ], wrg[WJ];
  auto fetch = [&](int k0) {
    if (!active) return;
#pragma unroll
    for (int j = 0; j < XJ; ++j) {
      const int i = tid + j * 256, r = i >> 4, c = (i & 15) * 4;
      xr[j] = t0 + r < T ? *reinterpret_cast<const v4f *>(x + (size_t)(t0 + r) * d + k0 + c)
                         : v4f{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < WJ; ++j) {
      const int i = tid + j * 256, r = i >> 4, c = (i & 15) * 4;
      wrg[j] = e0 + r < E ? *reinterpret_cast<const v4f *>(wr + (size_t)(e0 + r) * d + k0 + c)
                          : v4f{0.f, 0.f, 0.f, 0.f};
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < d; k0 += kRK) {
    if (active) {
#pragma unroll
      for (int j = 0; j < XJ; ++j) {
        const int i = tid + j * 256;
        *reinterpret_cast<v4f *>(xs + (i >> 4) * kRS + (i & 15) * 4) = xr[j];
      }
#pragma unroll
      for (int j = 0; j < WJ; ++j) {
        const int i = tid + j * 256;
        *reinterpret_cast<v4f *>(ws + (i >> 4) * kRS + (i & 15) * 4) = wrg[j];
      }
    }
    __syncthreads();
    if (k0 + kRK < d) fetch(k0 + kRK);
    if (active) {
      const float *xa = xs + (16 * th + lr) * kRS + lk;
      const float *wb0 = ws + (32 * eh + lr) * kRS + lk;
      const float *wb1 = wb0 + 16 * kRS;
#pragma unroll
      for (int kk = 0; kk < kRK; kk += 4) {
        const float a = xa[kk];
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, wb0[kk], acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, wb1[kk], acc[1], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  if (!active) return;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int e = e0 + 32 * eh + 16 * n + lr;
    if (e >= E) continue;
    const float b = bias ? bias[e] : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * th + 4 * lk + i;
      if (t < T) logits[(size_t)t * E + e] = bias ? acc[n][i] + b : acc[n][i];
    }
  }
}

// ------------------------------------------------------------------ top-k
// One wave per token.  Each expert's logit becomes an unsigned order key (its
// bits mapped so that unsigned order is float order, -0 folded onto +0; 0 is
// below every finite logit and marks a taken or absent expert).  k_t rounds
// pick the slots in order: a wave-wide max of the keys gives the largest
// logit, and a ballot of the lanes holding it gives the lowest expert index
// among equals (expert e sits in lane e % 64, slot e / 64).  The softmax over
// the picked logits is accumulated in slot order.
__device__ __forceinline__ uint32_t order_key(float l) {
  uint32_t b = __float_as_uint(l);
  if ((b & 0x7fffffffu) == 0) b = 0;  // -0 == +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// The logit an order key was made from (-0 comes back as +0, which gives the
// same exponentials below).
__device__ __forceinline__ float key_logit(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return (uint32_t)wave_reduce((int)v, [](int a, int b) {
    return (uint32_t)a > (uint32_t)b ? a : b;
  });
}

constexpr int kTopkSlots = kMaxExperts / kWave;

// NS slots of 64 experts per lane (E <= 64 * NS).
template <int NS>
__device__ __forceinline__ void topk_row_wave_n(const float *l, int E, int k_max, int kt,
                                                int32_t *__restrict__ ids_row,
                                                float *__restrict__ w_row, int lane) {
  // every slot's logit is requested before any is used (one memory latency)
  float lv[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    const int e = lane + c * kWave;
    lv[c] = c * kWave < E ? l[e < E ? e : E - 1] : 0.0f;
  }
  if constexpr (kDebugChecks) {
    bool fin = true;
#pragma unroll
    for (int c = 0; c < NS; ++c) fin &= !(lane + c * kWave < E) || __builtin_isfinite(lv[c]);
    dcheck(fin, kDbgNonFinite);
  }
  uint32_t key[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) key[c] = lane + c * kWave < E ? order_key(lv[c]) : 0u;
  float m = 0.0f, z = 0.0f, my_eps = 0.0f;
  int my_id = -1;
  for (int j = 0; j < kt; ++j) {
    uint32_t best = key[0];
#pragma unroll
    for (int c = 1; c < NS; ++c) best = key[c] > best ? key[c] : best;
    best = wave_max_u32(best);
    int e = -1;
#pragma unroll
    for (int c = 0; c < NS; ++c) {  // the lowest slot, then the lowest lane, holding the max
      const uint64_t hold = __ballot(key[c] == best);
      if (e < 0 && hold) e = c * kWave + (int)__builtin_ctzll(hold);
    }
    const float lg = key_logit(best);  // no dependent memory read per round
    if (j == 0) m = lg;
    const float eps = expf(lg - m);
    z += eps;
    if (lane == j) {
      my_eps = eps;
      my_id = e;
    }
    if ((e & 63) == lane) {
#pragma unroll
      for (int c = 0; c < NS; ++c)
        if (c == (e >> 6)) key[c] = 0u;
    }
  }
  if (lane < k_max) {
    ids_row[lane] = lane < kt ? my_id : -1;
    w_row[lane] = lane < kt ? my_eps / z : 0.0f;
  }
}

// More than 128 experts: lane l holds the NS consecutive experts NS*l ..
// NS*l + NS-1, sorted once (a sorting network on (key descending, index
// ascending)).  A pick is then one wave-wide max over the lanes' first keys
// and a ballot: among lanes holding the max the lowest lane has the lowest
// expert indices, and inside a lane equal keys are in index order, so the
// picks come in the same order as in topk_row_wave_n (logit descending, lower
// index first) -- the same ids and, accumulated in that order, the same
// weights -- for a few instructions per pick instead of a scan of every slot.
template <int NS>
__device__ __forceinline__ void topk_row_wave_sorted(const float *l, int E, int k_max, int kt,
                                                     int32_t *__restrict__ ids_row,
                                                     float *__restrict__ w_row, int lane) {
  uint32_t key[NS];
  int idx[NS];
  {
    float lv[NS];
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      const int e = lane * NS + c;
      lv[c] = e < E ? l[e] : 0.0f;
    }
    if constexpr (kDebugChecks) {
      bool fin = true;
#pragma unroll
      for (int c = 0; c < NS; ++c) fin &= !(lane * NS + c < E) || __builtin_isfinite(lv[c]);
      dcheck(fin, kDbgNonFinite);
    }
#pragma unroll
    for (int c = 0; c < NS; ++c) {
      const int e = lane * NS + c;
      key[c] = e < E ? order_key(lv[c]) : 0u;
      idx[c] = e;
    }
  }
  // slot i before slot j: larger key, or equal key and lower index
  auto cmpswap = [&](int i, int j) {
    const bool sw = key[j] > key[i] || (key[j] == key[i] && idx[j] < idx[i]);
    const uint32_t ki = key[i], kj = key[j];
    const int ii = idx[i], ij = idx[j];
    key[i] = sw ? kj : ki;
    key[j] = sw ? ki : kj;
    idx[i] = sw ? ij : ii;
    idx[j] = sw ? ii : ij;
  };
  static_assert(NS == 8, "the sorting network is the 19-comparator one for 8 inputs");
  cmpswap(0, 2); cmpswap(1, 3); cmpswap(4, 6); cmpswap(5, 7);
  cmpswap(0, 4); cmpswap(1, 5); cmpswap(2, 6); cmpswap(3, 7);
  cmpswap(0, 1); cmpswap(2, 3); cmpswap(4, 5); cmpswap(6, 7);
  cmpswap(2, 4); cmpswap(3, 5);
  cmpswap(1, 4); cmpswap(3, 6);
  cmpswap(1, 2); cmpswap(3, 4); cmpswap(5, 6);
  float m = 0.0f, z = 0.0f, my_eps = 0.0f;
  int my_id = -1;
  for (int j = 0; j < kt; ++j) {
    const uint32_t best = wave_max_u32(key[0]);
    const uint64_t hold = __ballot(key[0] == best);
    const int win = (int)__builtin_ctzll(hold);
    const int e = __builtin_amdgcn_readlane(idx[0], win);
    const bool pop = lane == win;  // the winner's list moves up by one
#pragma unroll
    for (int c = 0; c < NS - 1; ++c) {
      key[c] = pop ? key[c + 1] : key[c];
      idx[c] = pop ? idx[c + 1] : idx[c];
    }
    key[NS - 1] = pop ? 0u : key[NS - 1];
    const float lg = key_logit(best);
    if (j == 0) m = lg;
    const float eps = expf(lg - m);
    z += eps;
    if (lane == j) {
      my_eps = eps;
      my_id = e;
    }
  }
  if (lane < k_max) {
    ids_row[lane] = lane < kt ? my_id : -1;
    w_row[lane] = lane < kt ? my_eps / z : 0.0f;
  }
}

// l: the token's E logits (global memory or LDS); writes the token's k_max
// slots of ids / w.
__device__ __forceinline__ void topk_row_wave(const float *l, int E, int k_max, int kt,
                                              int32_t *__restrict__ ids_row,
                                              float *__restrict__ w_row, int lane) {
  if (E <= kWave)
    topk_row_wave_n<1>(l, E, k_max, kt, ids_row, w_row, lane);
  else if (E <= 2 * kWave)
    topk_row_wave_n<2>(l, E, k_max, kt, ids_row, w_row, lane);
  else
    topk_row_wave_sorted<kTopkSlots>(l, E, k_max, kt, ids_row, w_row, lane);
}

__device__ __forceinline__ void topk_token_wave(const float *__restrict__ logits, int T, int E,
                                                int k_max, const int32_t *__restrict__ kpt,
                                                int32_t *__restrict__ ids, float *__restrict__ w,
                                                int t, int lane) {
  (void)T;
  topk_row_wave(logits + (size_t)t * E, E, k_max, token_k(kpt, t, k_max), ids + (size_t)t * k_max,
                w + (size_t)t * k_max, lane);
}

// ------------------------------------------------------------------ routing, prefill-sized
// Batches with many tokens and at most 128 experts: one workgroup of eight
// waves takes TT = 2048/EW tokens against all experts (EW: E padded to 32, 64
// or 128), so each wave owns one 16 x 16 logit tile on v_mfma_f32_16x16x4_f32
// and every token is read by one workgroup only.  K advances 64 floats at a
// time through two LDS buffers (one barrier per chunk), the next chunk's
// global loads in flight while the current one is multiplied.  A lane reads
// its fragments as four 16-byte pieces: lane (r, q) feeds k = 16q + s to MFMA
// step s, the same k for both operands, so every product of the chunk is
// summed once.  The loading threads keep each token row's |x| maximum on the
// way; after the K loop the workgroup quantises its tokens (re-reading x) and,
// from the logits it keeps in LDS, picks their top-k with softmax weights.
// With xq == nullptr only the logits are written (moe_router_logits), with the
// same arithmetic, so the two give the same logits bit for bit.
constexpr int kRtChunk = 64, kRtStride = kRtChunk + 4, kRtThreads = 512, kRtPrefetch = 4;

// LDS bytes of one route tile of EW experts: two K buffers, the tile's
// logits and its tokens' |x| maxima.
template <int EW>
constexpr int route_tile_lds_bytes() {
  return (2 * (2048 / EW + EW) * kRtStride + (2048 / EW) * EW + 2048 / EW) * (int)sizeof(float);
}

// Tile (bx, by) of the routing grid (tokens [bx*TT, +TT), experts
// [by*EW, +EW)) by one workgroup of kRtThreads threads; lds: 16-byte aligned,
// route_tile_lds_bytes<EW>() bytes.
template <int EW>
__device__ __forceinline__ void route_tile_block(
    const float *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int T, int d, int E, int k_max, const int32_t *__restrict__ kpt, float *__restrict__ logits,
    uint8_t *__restrict__ xq, float *__restrict__ sx, int32_t *__restrict__ ids,
    float *__restrict__ w, int bx, int by, float *lds) {
  constexpr int TT = 2048 / EW, TB = TT / 16;
  constexpr int ROWS = TT + EW, NV = ROWS * 16, CJ = (NV + kRtThreads - 1) / kRtThreads;
  constexpr int XJ = (TT * 16 + kRtThreads - 1) / kRtThreads;  // staging slots holding x
  constexpr int PF = kRtPrefetch;
  static_assert(TB * (EW / 16) == kRtThreads / kWave, "one 16x16 tile per wave");
  float(*buf)[ROWS * kRtStride] = reinterpret_cast<float(*)[ROWS * kRtStride]>(lds);
  float *ls = lds + 2 * ROWS * kRtStride;
  float *ramax = ls + TT * EW;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t0 = bx * TT, e0 = by * EW;  // experts [e0, e0 + EW) of this block
  const int tb = wave % TB, eb = wave / TB;
  const int lr = lane & 15, lq = lane >> 4;
  const int nch = d / kRtChunk;
  // more than one expert block (E > EW): only block 0 quantises, top-k is left to the caller
  if (by != 0) xq = nullptr;

  // Each thread's staging slots: a fixed source row (clamped into range, so
  // every load is issued unconditionally and the wait counts stay exact) and
  // whether the row is real; chunk ch reads columns ch*64 + c .. +3.
  const float *src[CJ];
  bool real[CJ];
#pragma unroll
  for (int j = 0; j < CJ; ++j) {
    const int i = tid + j * kRtThreads, r = (i < NV ? i : NV - 1) >> 4, c = (i & 15) * 4;
    if (r < TT) {
      const int t = t0 + r;
      real[j] = i < NV && t < T;
      src[j] = x + (size_t)(t < T ? t : T - 1) * d + c;
    } else {
      const int e = e0 + r - TT;
      real[j] = i < NV && e < E;
      src[j] = wr + (size_t)(e < E ? e : E - 1) * d + c;
    }
  }
  v4f stg[PF][CJ];
  float amx[XJ];
#pragma unroll
  for (int j = 0; j < XJ; ++j) amx[j] = 0.0f;
  auto fetch = [&](v4f (&st)[CJ], int ch) {
    const int k0 = (ch < nch ? ch : nch - 1) * kRtChunk;  // past the end: reload the last chunk
#pragma unroll
    for (int j = 0; j < CJ; ++j) st[j] = *reinterpret_cast<const v4f *>(src[j] + k0);
  };
  auto put = [&](const v4f (&st)[CJ], float *b) {
#pragma unroll
    for (int j = 0; j < CJ; ++j) {
      const int i = tid + j * kRtThreads;
      const v4f v = real[j] ? st[j] : v4f{0.f, 0.f, 0.f, 0.f};
      if (i < NV) *reinterpret_cast<v4f *>(b + (i >> 4) * kRtStride + (i & 15) * 4) = v;
    }
#pragma unroll
    for (int j = 0; j < XJ; ++j)  // x rows come first: slots j < XJ
      if (tid + j * kRtThreads < TT * 16)
        amx[j] = fmaxf(amx[j], fmaxf(fmaxf(fabsf(st[j].x), fabsf(st[j].y)),
                                     fmaxf(fabsf(st[j].z), fabsf(st[j].w))));
  };

  v4f acc = {0.f, 0.f, 0.f, 0.f};
  // chunk c is loaded into stg[c % PF] at step c - PF + 1 and written to LDS
  // at the end of step c - 1
#pragma unroll
  for (int c = 0; c < PF - 1; ++c) fetch(stg[c], c);
  put(stg[0], buf[0]);
  __syncthreads();
  for (int ch0 = 0; ch0 < nch; ch0 += PF) {
#pragma unroll
    for (int s = 0; s < PF; ++s) {
      const int ch = ch0 + s;
      if (ch >= nch) break;
      fetch(stg[(s + PF - 1) % PF], ch + PF - 1);
      const float *b = buf[ch & 1];
      const float *xa = b + (tb * 16 + lr) * kRtStride + 16 * lq;
      const float *wb = b + (TT + eb * 16 + lr) * kRtStride + 16 * lq;
      v4f xv[4], wv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        xv[j] = *reinterpret_cast<const v4f *>(xa + 4 * j);
        wv[j] = *reinterpret_cast<const v4f *>(wb + 4 * j);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[j].x, wv[j].x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[j].y, wv[j].y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[j].z, wv[j].z, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xv[j].w, wv[j].w, acc, 0, 0, 0);
      }
      if (ch + 1 < nch) put(stg[(s + 1) % PF], buf[(ch + 1) & 1]);
      __syncthreads();
    }
  }

  // logits: tile rows are tokens, columns experts
  const int el = eb * 16 + lr, e = e0 + el;
  const float be = (bias && e < E) ? bias[e] : 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = tb * 16 + 4 * lq + i, t = t0 + r;
    const float lg = bias ? acc[i] + be : acc[i];
    ls[r * EW + el] = lg;
    if (t < T && e < E) logits[(size_t)t * E + e] = lg;
  }
  if (!xq) return;  // logits only, or an expert block past the first
  // each token row's |x| maximum: the 16 lanes that loaded it are one DPP row
#pragma unroll
  for (int j = 0; j < XJ; ++j) {
    float m = amx[j];
    m = fmaxf(m, dpp_mov<kDppQuadXor1>(m));
    m = fmaxf(m, dpp_mov<kDppQuadXor2>(m));
    m = fmaxf(m, dpp_mov<kDppHalfMirror>(m));
    m = fmaxf(m, dpp_mov<kDppMirror>(m));
    const int i = tid + j * kRtThreads;
    if (i < TT * 16 && (lane & 15) == 0) ramax[i >> 4] = m;
  }
  __syncthreads();
  // a wave per token: quantise it (re-reading x), then its top-k from LDS
  for (int r = wave; r < TT; r += kRtThreads / kWave) {
    const int t = t0 + r;
    if (t >= T) break;
    const float m = ramax[r];
    const float rq = m != 0.0f ? kE4m3Max / m : 1.0f;
    const float *xr = x + (size_t)t * d;
    uint8_t *q = xq + (size_t)t * d;
    for (int i0 = 0; i0 < d; i0 += 4 * kWave * 4) {
      v4f v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + (u * kWave + lane) * 4;
        v[u] = i < d ? *reinterpret_cast<const v4f *>(xr + i) : v4f{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + (u * kWave + lane) * 4;
        if (i < d) *reinterpret_cast<uint32_t *>(q + i) = e4m3x4(v[u].x * rq, v[u].y * rq, v[u].z * rq, v[u].w * rq);
      }
    }
    if (lane == 0) sx[t] = m != 0.0f ? m / kE4m3Max : 1.0f;
    if (ids)  // all experts in this block (E <= EW)
      topk_row_wave(ls + r * EW, E, k_max, token_k(kpt, t, k_max), ids + (size_t)t * k_max,
                    w + (size_t)t * k_max, lane);
  }
}

}  // namespace fp8moe
