// kernels_route.hip -- per-token e4m3 quantisation, fp32 router logits and
// wave64 top-k with softmax weights, for gfx950 (per-stage kernels; the
// device functions live in route_dev.hpp).
//
// Layer statement: "Routage MoE entre GPU" (router paragraph): the router
// scores every expert from the token's hidden state, keeps the best k and
// emits one routing weight per pick.  W8A8 FP8: Alpha-MoE article, opening
// section.
#include "common.hpp"
#include "internal.hpp"
#include "route_dev.hpp"

namespace fp8moe {
// ------------------------------------------------------------------ quantise
__global__ __launch_bounds__(256) void quantize_rows_kernel(const float *__restrict__ x, int rows,
                                                            int cols, uint8_t *__restrict__ q,
                                                            float *__restrict__ scale) {
  int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  quantize_row_wave(x + (size_t)row * cols, cols, q + (size_t)row * cols, scale + row,
                    threadIdx.x & 63);
}

// Rows up to 16384 values: a workgroup per row, the row in registers.
__global__ __launch_bounds__(256) void quantize_rows_block_kernel(const float *__restrict__ x,
                                                                  int cols, uint8_t *__restrict__ q,
                                                                  float *__restrict__ scale) {
  __shared__ float red[4];
  const size_t row = blockIdx.x;
  quantize_row_block<256, 16>(x + row * cols, cols, q + row * cols, scale + row, red);
}

hipError_t launch_quantize_rows(const float *x, int32_t rows, int32_t cols, uint8_t *q,
                                float *scale, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  if (cols <= 16384)
    quantize_rows_block_kernel<<<rows, 256, 0, stream>>>(x, cols, q, scale);
  else
    quantize_rows_kernel<<<(rows + 3) / 4, 256, 0, stream>>>(x, rows, cols, q, scale);
  return hipGetLastError();
}

// ------------------------------------------------------------------ router
// Batches of up to 65536 (token, expert) pairs: a wave takes two tokens x
// four experts and forms each of its eight dot products exactly as
// router_dot_wave does (the same lanes, the same order of FMAs, the same wave
// sum, the parts added in order), so the logits are the same bit for bit, while
// each x and W_r row is read once per wave instead of once per product.  The
// wave of the first four experts also quantises its tokens.
constexpr int kDotTok = 2, kDotExp = 4;
constexpr int64_t kRouterDotTileMin = 16384;  // (token, expert) pairs: from here the tiled form

__global__ __launch_bounds__(256) void router_dot_tile_kernel(const float *__restrict__ x,
                                                              const float *__restrict__ wr,
                                                              const float *__restrict__ bias, int T,
                                                              int d, int E,
                                                              float *__restrict__ logits,
                                                              uint8_t *__restrict__ xq,
                                                              float *__restrict__ sx) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int n_eq = (E + kDotExp - 1) / kDotExp;
  const int tp = wid / n_eq, eq = wid - tp * n_eq;
  const int t0 = tp * kDotTok, e0 = eq * kDotExp;
  if (t0 >= T) return;
  float logit[kDotTok][kDotExp], amax[kDotTok];
#pragma unroll
  for (int u = 0; u < kDotTok; ++u) amax[u] = 0.0f;
  v4f xv[kDotTok][kDotVec];
  for (int base = 0; base < d; base += kDotPart) {
    v4f wv[kDotExp][kDotVec];
#pragma unroll
    for (int j = 0; j < kDotVec; ++j) {
      const int i = base + (j * 64 + lane) * 4;
#pragma unroll
      for (int u = 0; u < kDotTok; ++u)
        xv[u][j] = (i < d && t0 + u < T) ? *reinterpret_cast<const v4f *>(x + (size_t)(t0 + u) * d + i)
                                         : v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < kDotExp; ++v)
        wv[v][j] = (i < d && e0 + v < E) ? *reinterpret_cast<const v4f *>(wr + (size_t)(e0 + v) * d + i)
                                         : v4f{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kDotTok; ++u) {
#pragma unroll
      for (int j = 0; j < kDotVec; ++j)
        amax[u] = fmaxf(amax[u], fmaxf(fmaxf(fabsf(xv[u][j].x), fabsf(xv[u][j].y)),
                                       fmaxf(fabsf(xv[u][j].z), fabsf(xv[u][j].w))));
#pragma unroll
      for (int v = 0; v < kDotExp; ++v) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < kDotVec; ++j) {
          acc = fmaf(xv[u][j].x, wv[v][j].x, acc);
          acc = fmaf(xv[u][j].y, wv[v][j].y, acc);
          acc = fmaf(xv[u][j].z, wv[v][j].z, acc);
          acc = fmaf(xv[u][j].w, wv[v][j].w, acc);
        }
        const float ps = wave_sum(acc);
        logit[u][v] = base == 0 ? ps : logit[u][v] + ps;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kDotTok; ++u) {
    const int t = t0 + u;
    if (t >= T) break;
#pragma unroll
    for (int v = 0; v < kDotExp; ++v) {
      const int e = e0 + v;
      if (e < E && lane == 0) logits[(size_t)t * E + e] = bias ? logit[u][v] + bias[e] : logit[u][v];
    }
    if (eq == 0 && xq) {
      const float m = wave_max(amax[u]);
      uint8_t *q = xq + (size_t)t * d;
      if (d <= kDotPart) {
        quantize_part_wave(xv[u], d, 0, m, q, lane);
      } else {
        const float r = m != 0.0f ? kE4m3Max / m : 1.0f;
        const float *xr = x + (size_t)t * d;
        for (int i = lane * 4; i < d; i += kWave * 4) {
          const v4f v = *reinterpret_cast<const v4f *>(xr + i);
          *reinterpret_cast<uint32_t *>(q + i) = e4m3x4(v.x * r, v.y * r, v.z * r, v.w * r);
        }
      }
      if (lane == 0) sx[t] = m != 0.0f ? m / kE4m3Max : 1.0f;
    }
  }
}

// Small batches: one wave per (token, expert) product keeps more waves in flight.
__global__ __launch_bounds__(256) void router_dot_kernel(const float *__restrict__ x,
                                                         const float *__restrict__ wr,
                                                         const float *__restrict__ bias, int T,
                                                         int d, int E, float *__restrict__ logits,
                                                         uint8_t *__restrict__ xq,
                                                         float *__restrict__ sx) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= T * E) return;
  const int t = wid / E;
  router_dot_wave(x, wr, bias, d, E, logits, xq, sx, t, wid - t * E, threadIdx.x & 63);
}

static hipError_t launch_router_dot(const float *x, const float *w_router, const float *bias,
                                    int32_t T, int32_t d, int32_t E, float *logits, uint8_t *xq,
                                    float *sx, hipStream_t stream) {
  if ((int64_t)T * E < kRouterDotTileMin) {
    router_dot_kernel<<<(T * E + 3) / 4, 256, 0, stream>>>(x, w_router, bias, T, d, E, logits, xq,
                                                           sx);
    return hipGetLastError();
  }
  const int64_t waves = (int64_t)((T + kDotTok - 1) / kDotTok) * ((E + kDotExp - 1) / kDotExp);
  router_dot_tile_kernel<<<(int)((waves + 3) / 4), 256, 0, stream>>>(x, w_router, bias, T, d, E,
                                                                     logits, xq, sx);
  return hipGetLastError();
}

// Decode-sized batches: one workgroup per token computes its E logits (the
// arithmetic of router_dot_wave, so the logits equal those of
// moe_router_logits), quantises the token and, from the logits kept in LDS,
// picks its top-k with softmax weights -- routing in one launch.  With
// E * parts(d) <= 16 every (expert, part) has a wave of its own and the
// token is quantised from the registers of expert 0's waves; otherwise each
// wave walks its experts' parts.
constexpr int kRouteWaves = 16;
constexpr int kMaxDotParts = kRouteWaves;

__global__ __launch_bounds__(kRouteWaves * kWave) void route_token_kernel(
    const float *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int d, int E, int k_max, const int32_t *__restrict__ kpt, float *__restrict__ logits,
    uint8_t *__restrict__ xq, float *__restrict__ sx, int32_t *__restrict__ ids,
    float *__restrict__ w) {
  __shared__ float ls[kMaxExperts];
  __shared__ float psum[kRouteWaves], pmax[kMaxDotParts];
  const int t = blockIdx.x, lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int parts = (d + kDotPart - 1) / kDotPart;
  if (E * parts <= nw) {
    const int e = wave / parts, part = wave - e * parts;  // wave-uniform
    v4f xv[kDotVec];
    if (e < E) {
      float amax = 0.0f;
      const float ps = router_part_wave(x + (size_t)t * d, wr + (size_t)e * d, d,
                                        part * kDotPart, lane, xv, amax);
      if (lane == 0) psum[wave] = ps;
      if (e == 0) {
        amax = wave_max(amax);
        if (lane == 0) pmax[part] = amax;
      }
    }
    __syncthreads();
    if (e == 0 && xq) {  // expert 0's waves quantise their parts of the token from registers
      float m = pmax[0];
      for (int p = 1; p < parts; ++p) m = fmaxf(m, pmax[p]);
      quantize_part_wave(xv, d, part * kDotPart, m, xq + (size_t)t * d, lane);
      if (wave == 0 && lane == 0) sx[t] = m != 0.0f ? m / kE4m3Max : 1.0f;
    }
    // part sums in part order, as router_dot_wave adds them
    for (int ee = threadIdx.x; ee < E; ee += blockDim.x) {
      float lg = psum[ee * parts];
      for (int p = 1; p < parts; ++p) lg = lg + psum[ee * parts + p];
      if (bias) lg += bias[ee];
      ls[ee] = lg;
      logits[(size_t)t * E + ee] = lg;
    }
  } else {
    for (int e = wave; e < E; e += nw) {
      const float lg = router_dot_wave(x, wr, bias, d, E, logits, xq, sx, t, e, lane);
      if (lane == 0) ls[e] = lg;
    }
  }
  __syncthreads();
  if (wave == 0)
    topk_row_wave(ls, E, k_max, token_k(kpt, t, k_max), ids + (size_t)t * k_max,
                  w + (size_t)t * k_max, lane);
}

// One workgroup per token pays off while a token's experts fit one wave each.
bool route_fused_applies(int32_t T, int32_t E) {
  return E <= kRouteWaves && (int64_t)T * E <= kRouterDotMax;
}

hipError_t launch_route_topk_fused(const float *x, const float *w_router, const float *bias,
                                   int32_t T, int32_t d, int32_t E, int32_t k_max,
                                   const int32_t *kpt, float *logits, uint8_t *xq, float *sx,
                                   int32_t *ids, float *w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  // a wave per (expert, part) where they fit, else a wave per expert
  const int parts = (d + kDotPart - 1) / kDotPart;
  const int nw = E * parts <= kRouteWaves ? E * parts : (E < kRouteWaves ? E : kRouteWaves);
  route_token_kernel<<<T, nw * 64, 0, stream>>>(x, w_router, bias, d, E, k_max, kpt, logits, xq,
                                                sx, ids, w);
  return hipGetLastError();
}

// ------------------------------------------------------------------ routing, prefill-sized
// (route_tile_block in route_dev.hpp)
template <int EW>
__global__ __launch_bounds__(kRtThreads) void route_tile_kernel(
    const float *__restrict__ x, const float *__restrict__ wr, const float *__restrict__ bias,
    int T, int d, int E, int k_max, const int32_t *__restrict__ kpt, float *__restrict__ logits,
    uint8_t *__restrict__ xq, float *__restrict__ sx, int32_t *__restrict__ ids,
    float *__restrict__ w) {
  __shared__ __attribute__((aligned(16))) float lds[route_tile_lds_bytes<EW>() / sizeof(float)];
  route_tile_block<EW>(x, wr, bias, T, d, E, k_max, kpt, logits, xq, sx, ids, w, blockIdx.x,
                       blockIdx.y, lds);
}

// Prefill-sized batches route in one launch (logits, quantised x, top-k).
bool route_tile_applies(int32_t T, int32_t E) {
  return E <= 128 && (int64_t)T * E > kRouterDotMax;
}

static hipError_t launch_route_tile(const float *x, const float *w_router, const float *bias,
                                    int32_t T, int32_t d, int32_t E, int32_t k_max,
                                    const int32_t *kpt, float *logits, uint8_t *xq, float *sx,
                                    int32_t *ids, float *w, hipStream_t stream) {
  if (E <= 32)
    route_tile_kernel<32><<<(T + 63) / 64, kRtThreads, 0, stream>>>(x, w_router, bias, T, d, E, k_max, kpt, logits, xq, sx, ids, w);
  else if (E <= 64)
    route_tile_kernel<64><<<(T + 31) / 32, kRtThreads, 0, stream>>>(x, w_router, bias, T, d, E, k_max, kpt, logits, xq, sx, ids, w);
  else  // E > 128: blocks of 128 experts along y; the caller runs the top-k
    route_tile_kernel<128><<<dim3((T + 15) / 16, (E + 127) / 128), kRtThreads, 0, stream>>>(
        x, w_router, bias, T, d, E, k_max, kpt, logits, xq, sx, E <= 128 ? ids : nullptr, w);
  return hipGetLastError();
}

hipError_t launch_route_prefill(const float *x, const float *w_router, const float *bias,
                                int32_t T, int32_t d, int32_t E, int32_t k_max,
                                const int32_t *kpt, float *logits, uint8_t *xq, float *sx,
                                int32_t *ids, float *w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  return launch_route_tile(x, w_router, bias, T, d, E, k_max, kpt, logits, xq, sx, ids, w, stream);
}

hipError_t launch_route_logits(const float *x, const float *w_router, const float *bias, int32_t T,
                               int32_t d, int32_t E, float *logits, uint8_t *xq, float *sx,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if ((int64_t)T * E <= kRouterDotMax)
    return launch_router_dot(x, w_router, bias, T, d, E, logits, xq, sx, stream);
  if (E > 128)  // the tiled router over expert blocks, quantising x in its first block
    return launch_route_tile(x, w_router, bias, T, d, E, 0, nullptr, logits, xq, sx, nullptr,
                             nullptr, stream);
  hipError_t e = hipSuccess;
  if (xq && (e = launch_quantize_rows(x, T, d, xq, sx, stream)) != hipSuccess) return e;
  return launch_router(x, w_router, bias, T, d, E, logits, stream);
}

hipError_t launch_router(const float *x, const float *w_router, const float *bias, int32_t T,
                         int32_t d, int32_t E, float *logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if ((int64_t)T * E <= kRouterDotMax)
    return launch_router_dot(x, w_router, bias, T, d, E, logits, nullptr, nullptr, stream);
  // the arithmetic of the fused routing (one expert block, or blocks of 128)
  return launch_route_tile(x, w_router, bias, T, d, E, 0, nullptr, logits, nullptr, nullptr,
                           nullptr, nullptr, stream);
}

// ------------------------------------------------------------------ top-k
__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k_max, const int32_t *__restrict__ kpt,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  topk_token_wave(logits, T, E, k_max, kpt, ids, w, t, threadIdx.x & 63);
}

hipError_t launch_topk(const float *logits, int32_t T, int32_t E, int32_t k_max,
                       const int32_t *k_per_token, int32_t *ids, float *w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  topk_kernel<<<(T + 3) / 4, 256, 0, stream>>>(logits, T, E, k_max, k_per_token, ids, w);
  return hipGetLastError();
}

// Debug build: this file's device-check word (see common.hpp).
FP8MOE_DEBUG_TAKE(route)

}  // namespace fp8moe
