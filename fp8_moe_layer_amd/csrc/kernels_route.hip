// kernels_route.hip -- per-token e4m3 quantisation, fp32 router logits and
// wave64 top-k with softmax weights, for gfx950.
//
// Layer statement: "Routage MoE entre GPU" (router paragraph): the router
// scores every expert from the token's hidden state, keeps the best k and
// emits one routing weight per pick.  W8A8 FP8: Alpha-MoE article, opening
// section.
#include "common.hpp"
#include "internal.hpp"

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

// ------------------------------------------------------------------ router, decode-sized
// One wave per (token, expert) dot product over d, lanes striding d by 4
// floats with all of a lane's loads issued before the FMAs.  The wave of
// expert 0 also quantises its token's row (it has read the row already).
constexpr int kDotVec = 8;  // float4 per lane per round: d <= 2048 in one round

__global__ __launch_bounds__(256) void router_dot_kernel(const float *__restrict__ x,
                                                         const float *__restrict__ wr,
                                                         const float *__restrict__ bias, int T,
                                                         int d, int E, float *__restrict__ logits,
                                                         uint8_t *__restrict__ xq,
                                                         float *__restrict__ sx) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= T * E) return;
  const int lane = threadIdx.x & 63;
  const int t = wid / E, e = wid - t * E;
  const float *xr = x + (size_t)t * d;
  const float *w = wr + (size_t)e * d;
  float acc = 0.0f, amax = 0.0f;
  for (int base = 0; base < d; base += kDotVec * 256) {
    v4f xv[kDotVec], wv[kDotVec];
#pragma unroll
    for (int j = 0; j < kDotVec; ++j) {
      const int i = base + (j * 64 + lane) * 4;
      xv[j] = i < d ? *reinterpret_cast<const v4f *>(xr + i) : v4f{0.f, 0.f, 0.f, 0.f};
      wv[j] = i < d ? *reinterpret_cast<const v4f *>(w + i) : v4f{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int j = 0; j < kDotVec; ++j) {
      acc = fmaf(xv[j].x, wv[j].x, acc);
      acc = fmaf(xv[j].y, wv[j].y, acc);
      acc = fmaf(xv[j].z, wv[j].z, acc);
      acc = fmaf(xv[j].w, wv[j].w, acc);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(xv[j].x), fabsf(xv[j].y)),
                               fmaxf(fabsf(xv[j].z), fabsf(xv[j].w))));
    }
  }
  acc = wave_sum(acc);
  if (lane == 0) logits[(size_t)t * E + e] = bias ? acc + bias[e] : acc;
  if (e == 0 && xq) {
    amax = wave_max(amax);
    float r = 1.0f, s = 1.0f;
    if (amax != 0.0f) {
      r = kE4m3Max / amax;
      s = amax / kE4m3Max;
    }
    uint8_t *q = xq + (size_t)t * d;
    for (int i = lane * 4; i < d; i += kWave * 4) {
      const v4f v = *reinterpret_cast<const v4f *>(xr + i);
      *reinterpret_cast<uint32_t *>(q + i) = e4m3x4(v.x * r, v.y * r, v.z * r, v.w * r);
    }
    if (lane == 0) sx[t] = s;
  }
}

hipError_t launch_route_logits(const float *x, const float *w_router, const float *bias, int32_t T,
                               int32_t d, int32_t E, float *logits, uint8_t *xq, float *sx,
                               hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if ((int64_t)T * E <= kRouterDotMax) {
    router_dot_kernel<<<(T * E + 3) / 4, 256, 0, stream>>>(x, w_router, bias, T, d, E, logits, xq,
                                                           sx);
    return hipGetLastError();
  }
  hipError_t e = hipSuccess;
  if (xq && (e = launch_quantize_rows(x, T, d, xq, sx, stream)) != hipSuccess) return e;
  return launch_router(x, w_router, bias, T, d, E, logits, stream);
}

// ------------------------------------------------------------------ router, tiled
// logits[t][e] = x[t] . w_router[e] (+ bias[e]) in fp32.  A workgroup takes
// TT tokens (kept in LDS) and a block of experts; each wave owns experts
// e = block + wave, +4, ... and reduces TT dot products over d.
template <int TT>
__global__ __launch_bounds__(256) void router_kernel(const float *__restrict__ x,
                                                     const float *__restrict__ wr,
                                                     const float *__restrict__ bias, int T, int d,
                                                     int E, int eb, float *__restrict__ logits) {
  extern __shared__ float xs[];  // [TT][d]
  const int t0 = blockIdx.x * TT;
  const int nt = min(TT, T - t0);
  for (int i = threadIdx.x * 4; i < TT * d; i += 256 * 4) {
    int tt = i / d;
    v4f v = {0.f, 0.f, 0.f, 0.f};
    if (tt < nt) v = *reinterpret_cast<const v4f *>(x + (size_t)t0 * d + i);
    *reinterpret_cast<v4f *>(xs + i) = v;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int e0 = blockIdx.y * eb;
  const int e1 = min(E, e0 + eb);
  for (int e = e0 + wave; e < e1; e += 4) {
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.0f;
    const float *w = wr + (size_t)e * d;
    for (int i = lane * 4; i < d; i += kWave * 4) {
      v4f wv = *reinterpret_cast<const v4f *>(w + i);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        v4f xv = *reinterpret_cast<const v4f *>(xs + t * d + i);
        acc[t] = fmaf(wv.x, xv.x, acc[t]);
        acc[t] = fmaf(wv.y, xv.y, acc[t]);
        acc[t] = fmaf(wv.z, xv.z, acc[t]);
        acc[t] = fmaf(wv.w, xv.w, acc[t]);
      }
    }
    float mine = 0.0f;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float s = wave_sum(acc[t]);
      if (lane == t) mine = s;
    }
    if (lane < nt) {
      if (bias) mine += bias[e];
      logits[(size_t)(t0 + lane) * E + e] = mine;
    }
  }
}

hipError_t launch_router(const float *x, const float *w_router, const float *bias, int32_t T,
                         int32_t d, int32_t E, float *logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  if ((int64_t)T * E <= kRouterDotMax) {
    router_dot_kernel<<<(T * E + 3) / 4, 256, 0, stream>>>(x, w_router, bias, T, d, E, logits,
                                                           nullptr, nullptr);
    return hipGetLastError();
  }
  // keep the token tile at <= 64 KB of LDS
  int tt = 16384 / d;
  int eb = E <= 64 ? E : 64;
  dim3 block(256);
  if (tt >= 16) {
    dim3 grid((T + 15) / 16, (E + eb - 1) / eb);
    router_kernel<16><<<grid, block, 16 * d * sizeof(float), stream>>>(x, w_router, bias, T, d, E,
                                                                        eb, logits);
  } else if (tt >= 8) {
    dim3 grid((T + 7) / 8, (E + eb - 1) / eb);
    router_kernel<8><<<grid, block, 8 * d * sizeof(float), stream>>>(x, w_router, bias, T, d, E, eb,
                                                                      logits);
  } else if (tt >= 4) {
    dim3 grid((T + 3) / 4, (E + eb - 1) / eb);
    router_kernel<4><<<grid, block, 4 * d * sizeof(float), stream>>>(x, w_router, bias, T, d, E, eb,
                                                                      logits);
  } else {
    dim3 grid(T, (E + eb - 1) / eb);
    router_kernel<1><<<grid, block, d * sizeof(float), stream>>>(x, w_router, bias, T, d, E, eb,
                                                                  logits);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-k
// One wave per token.  Each expert becomes a 64-bit key: the logit's bits
// mapped to an unsigned order (with -0 folded onto +0) in the high word and
// 0xFFFF - e in the low word, so the largest key is the largest logit with
// the lowest index.  k_t rounds of a wave-wide max pick the slots in order;
// the softmax over the picked logits is accumulated in slot order.
__device__ __forceinline__ uint64_t route_key(float l, int e) {
  uint32_t b = __float_as_uint(l);
  if ((b & 0x7fffffffu) == 0) b = 0;  // -0 == +0
  uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)(0xFFFF - e);
}

constexpr int kTopkSlots = kMaxExperts / kWave;

__global__ __launch_bounds__(256) void topk_kernel(const float *__restrict__ logits, int T, int E,
                                                   int k_max, const int32_t *__restrict__ kpt,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const float *l = logits + (size_t)t * E;
  uint64_t key[kTopkSlots];
#pragma unroll
  for (int c = 0; c < kTopkSlots; ++c) {
    int e = lane + c * kWave;
    key[c] = e < E ? route_key(l[e], e) : 0ull;
  }
  const int kt = kpt ? kpt[t] : k_max;
  float m = 0.0f, z = 0.0f, my_eps = 0.0f;
  int my_id = -1;
  for (int j = 0; j < kt; ++j) {
    uint64_t best = 0;
#pragma unroll
    for (int c = 0; c < kTopkSlots; ++c) best = key[c] > best ? key[c] : best;
    best = wave_max_u64(best);
    const int e = 0xFFFF - (int)(best & 0xFFFFu);
    const float lv = l[e];
    if (j == 0) m = lv;
    const float eps = expf(lv - m);
    z += eps;
    if (lane == j) {
      my_eps = eps;
      my_id = e;
    }
    if ((e & 63) == lane) {
#pragma unroll
      for (int c = 0; c < kTopkSlots; ++c)
        if (c == (e >> 6)) key[c] = 0ull;
    }
  }
  if (lane < k_max) {
    const size_t o = (size_t)t * k_max + lane;
    ids[o] = lane < kt ? my_id : -1;
    w[o] = lane < kt ? my_eps / z : 0.0f;
  }
}

hipError_t launch_topk(const float *logits, int32_t T, int32_t E, int32_t k_max,
                       const int32_t *k_per_token, int32_t *ids, float *w, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  topk_kernel<<<(T + 3) / 4, 256, 0, stream>>>(logits, T, E, k_max, k_per_token, ids, w);
  return hipGetLastError();
}

}  // namespace fp8moe
