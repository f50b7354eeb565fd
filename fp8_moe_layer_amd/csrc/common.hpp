// common.hpp -- device helpers shared by the gfx950 kernels of the FP8 MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxExperts = 512;  // routed experts per layer (top-k keys, permutation LDS)
constexpr int kMaxK = 32;         // slots per token
constexpr int kMaxFfn = 16384;  // longest h row the requantisation holds in registers
constexpr float kE4m3Max = 448.0f;

// ---------------------------------------------------------------- debug checks
// Built with FP8MOE_DEBUG (libfp8moe_debug.so), the kernels test the layer's
// preconditions and index invariants as they go.  A failed check sets its
// bit in a device word of the kernel's translation unit (an atomic OR
// through the vector memory path), and the failing value is replaced by a
// safe one (a clamped k, a dropped id, a skipped row), so a failed check
// never becomes an out-of-bounds access.  After each entry point the host
// collects and clears the words (debug_take_*).  In the release library
// dcheck() only returns its condition (the safe replacement still applies;
// checks that cost more than a compare are compiled in only when debugging).
enum : uint32_t {
  kDbgKPerToken = 1u << 0,  // k_per_token[t] outside [1, k_max]
  kDbgNonFinite = 1u << 1,  // a non-finite router logit, or a non-finite row to quantise
  kDbgTopkId = 1u << 2,     // a top-k id outside [-1, E)
  kDbgPermute = 1u << 3,    // a work item outside the expert row space
  kDbgRow = 1u << 4,        // a sorted pair or combine row index outside its range
  kDbgTile = 1u << 5,       // a GEMM wave's first weight channel not a multiple of 16
};
#ifdef FP8MOE_DEBUG
constexpr bool kDebugChecks = true;
static __device__ uint32_t g_debug_bits;  // one word per translation unit
__device__ __forceinline__ bool dcheck(bool ok, uint32_t bit) {
  if (!ok) atomicOr(&g_debug_bits, bit);
  return ok;
}
// Host: this translation unit's word, then cleared (the device is synchronised first).
#define FP8MOE_DEBUG_TAKE(NAME)                                                            \
  uint32_t debug_take_##NAME() {                                                           \
    uint32_t v = 0, z = 0;                                                                 \
    if (hipDeviceSynchronize() != hipSuccess ||                                            \
        hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_bits), sizeof v, 0,                     \
                            hipMemcpyDeviceToHost) != hipSuccess)                          \
      return 0x80000000u;                                                                  \
    if (v && hipMemcpyToSymbol(HIP_SYMBOL(g_debug_bits), &z, sizeof z, 0,                  \
                               hipMemcpyHostToDevice) != hipSuccess)                       \
      return v | 0x80000000u;                                                              \
    return v;                                                                              \
  }
#else
constexpr bool kDebugChecks = false;
__device__ __forceinline__ bool dcheck(bool ok, uint32_t) { return ok; }
#define FP8MOE_DEBUG_TAKE(NAME) \
  uint32_t debug_take_##NAME() { return 0; }
#endif

// k of token t: k_per_token[t], clamped to [1, k_max] (the debug build
// records a value outside it), or k_max without a per-token array.
__device__ __forceinline__ int token_k(const int32_t *kpt, int t, int k_max) {
  if (!kpt) return k_max;
  const int k = kpt[t];
  return dcheck(k >= 1 && k <= k_max, kDbgKPerToken) ? k : (k < 1 ? 1 : k_max);
}

// A top-k id as the permutation reads it: an id outside [-1, E) is dropped
// (-1; the debug build records it).
__device__ __forceinline__ int checked_id(int e, int E) {
  return dcheck(e >= -1 && e < E, kDbgTopkId) ? e : -1;
}

// ---------------------------------------------------------------- e4m3 codec
// gfx950's v_cvt_pk_fp8_f32 converts to OCP E4M3FN with round-to-nearest-even.
// Inputs are clamped to +-448 first, which is the saturating rule for every
// finite input (NaN inputs are outside the library's preconditions).
__device__ __forceinline__ float sat448(float v) { return fminf(fmaxf(v, -kE4m3Max), kE4m3Max); }

// Four floats -> four e4m3 codes packed little-endian in one 32-bit word.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), w, true);
  return (uint32_t)w;
}

// Two e4m3 codes (bytes 0,1 or, with HI, bytes 2,3 of a word) -> two floats, exact.
template <bool HI>
__device__ __forceinline__ v2f e4m3x2_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

// ---------------------------------------------------------------- MFMA
// D = A * B^T + C on a 16x16 fp32 tile with K = 128 e4m3 values.
// Lane l supplies row (l % 16) of A and row (l % 16) of B (B given with K
// contiguous, i.e. as the N x K weight matrix), 32 bytes of K each; the same
// K bytes must be supplied for A and B in the same lane.  Result: lane l,
// element i holds C[4 * (l / 16) + i][l % 16].
__device__ __forceinline__ v4f mfma_e4m3_16x16x128(v8i a, v8i b, v4f c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Same tile shape on fp16 operands with K = 32 (8 halves per lane).
__device__ __forceinline__ v4f mfma_f16_16x16x32(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave reductions
// Cross-lane steps inside each row of 16 lanes use DPP (a register operand
// modifier, a few cycles) rather than ds_bpermute (a round trip through the
// LDS crossbar); the four row results are then combined from v_readlane
// values, identically in every lane.  All 64 lanes must be active.
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within each half row
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within each row
constexpr int kDppRowShr = 0x110;     // + n: lane i reads lane i - n of its row (n = 1..15)

template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(dpp_mov<CTRL>(__float_as_int(v)));
}

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float readlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// Butterfly inside each row of 16 (every lane of a row ends with the row's
// result; op must be commutative), then the rows in the order (0,1),(2,3).
template <class T, class Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp_mov<kDppQuadXor1>(v));
  v = op(v, dpp_mov<kDppQuadXor2>(v));
  v = op(v, dpp_mov<kDppHalfMirror>(v));
  v = op(v, dpp_mov<kDppMirror>(v));
  return op(op(readlane(v, 0), readlane(v, 16)), op(readlane(v, 32), readlane(v, 48)));
}

__device__ __forceinline__ float wave_max(float v) {
  return wave_reduce(v, [](float a, float b) { return fmaxf(a, b); });
}

// The sum comes out bitwise the same in every lane.
__device__ __forceinline__ float wave_sum(float v) {
  return wave_reduce(v, [](float a, float b) { return a + b; });
}


// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 2, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 4, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kDppRowShr + 8, 0xf, 0xf, false);
  const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
            r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = lane >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ bool finite4(v4f v) {
  return __builtin_isfinite(v.x) && __builtin_isfinite(v.y) && __builtin_isfinite(v.z) &&
         __builtin_isfinite(v.w);
}

// ---------------------------------------------------------------- row quantisation
// One wave per row.  amax over the row, r = 448/amax and s = amax/448 as two
// correctly rounded fp32 divisions, codes = e4m3(x * r).  The same IEEE
// operations as the plain definition, so codes and scales are bit-exact.
__device__ __forceinline__ void quantize_row_wave(const float *__restrict__ x, int cols,
                                                  uint8_t *__restrict__ q, float *scale,
                                                  int lane) {
  float amax = 0.0f;
  for (int i = lane * 4; i < cols; i += kWave * 4) {
    v4f v = *reinterpret_cast<const v4f *>(x + i);
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    if constexpr (kDebugChecks) dcheck(finite4(v), kDbgNonFinite);
  }
  amax = wave_max(amax);
  float r = 1.0f, s = 1.0f;
  if (amax != 0.0f) {
    r = kE4m3Max / amax;
    s = amax / kE4m3Max;
  }
  for (int i = lane * 4; i < cols; i += kWave * 4) {
    v4f v = *reinterpret_cast<const v4f *>(x + i);
    *reinterpret_cast<uint32_t *>(q + i) = e4m3x4(v.x * r, v.y * r, v.z * r, v.w * r);
  }
  if (lane == 0) *scale = s;
}

// One workgroup of NT threads per row, the row held in registers between the
// max and the conversion (cols <= NT * 4 * VEC, cols a multiple of 4).  The
// same IEEE operations as quantize_row_wave; `red` is NT/64 floats of LDS.
template <int NT, int VEC>
__device__ __forceinline__ void quantize_row_block(const float *__restrict__ x, int cols,
                                                   uint8_t *__restrict__ q, float *scale,
                                                   float *red) {
  v4f v[VEC];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const int i = (j * NT + (int)threadIdx.x) * 4;
    v[j] = i < cols ? *reinterpret_cast<const v4f *>(x + i) : v4f{0.f, 0.f, 0.f, 0.f};
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    if constexpr (kDebugChecks) dcheck(finite4(v[j]), kDbgNonFinite);
  }
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = red[0];
#pragma unroll
  for (int w = 1; w < NT / kWave; ++w) amax = fmaxf(amax, red[w]);
  float r = 1.0f, s = 1.0f;
  if (amax != 0.0f) {
    r = kE4m3Max / amax;
    s = amax / kE4m3Max;
  }
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const int i = (j * NT + (int)threadIdx.x) * 4;
    if (i < cols)
      *reinterpret_cast<uint32_t *>(q + i) = e4m3x4(v[j].x * r, v[j].y * r, v[j].z * r, v[j].w * r);
  }
  if (threadIdx.x == 0) *scale = s;
}

// ---------------------------------------------------------------- memory
__device__ __forceinline__ v4i load16(const void *p) { return *reinterpret_cast<const v4i *>(p); }

__device__ __forceinline__ v4i load16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

}  // namespace fp8moe
