// kernels_expert.hip -- expert FFN stages of the W8A8 FP8 MoE layer on gfx950:
// gate/up grouped GEMM with the SiLU*up epilogue, per-row e4m3
// requantisation, down-projection grouped GEMM, and the weighted combine.
//
// "Routage MoE entre GPU": each expert is a feed-forward network with its
// own weights and only the selected experts process a token; the outputs are
// weighted, summed and put back in token order.  W8A8 FP8: Alpha-MoE article,
// opening section.
//
// Grouped GEMM schedule (weight-stationary).  A workgroup owns one work item
// (an expert and up to a chunk of that expert's rows) and one tile of output
// channels; it streams that tile's weight rows from HBM exactly once per pass
// of up to 16*MSUB rows and multiplies them against every row of the pass.
// Decode-sized batches fit all rows of an expert in one pass, so each active
// expert's weights cross HBM once.  Each wave owns 16 output channels (two
// weight rows per lane for gate/up, `kDownSub` row groups for down) and runs
// v_mfma_f32_16x16x128_f8f6f4 on e4m3 operands read straight from global
// memory into the MFMA lane layout: lane l supplies row l%16 and the 32
// K-bytes [32*(l/16), 32*(l/16)+32) of every 128-wide K step, for both the
// activation row and the weight row.
#include "common.hpp"
#include "internal.hpp"

namespace fp8moe {

namespace {

struct GemmArgs {
  RowSpace rs;
  const uint8_t *a;      // gate/up: xq [T][d]; down: hq [rows][f]
  const float *a_scale;  // sx [T] or sh [rows]
  const float *a32;      // down, fp32 mode: h [rows][f]
  ExpertWeights w;
  float *out;            // h [rows][f] or y [rows][d]
};

__device__ __forceinline__ v8i load32(const uint8_t *p) {
  const v4i lo = *reinterpret_cast<const v4i *>(p);
  const v4i hi = *reinterpret_cast<const v4i *>(p + 16);
  return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

__device__ __forceinline__ bool resolve_item(const RowSpace &rs, int item_id, int &expert,
                                             int &row0, int &rows) {
  if (rs.items) {
    if (item_id >= *rs.n_items) return false;
    const WorkItem it = rs.items[item_id];
    expert = it.expert;
    row0 = it.row0;
    rows = it.rows;
  } else {
    expert = item_id;
    if (expert < rs.E) {
      row0 = rs.expert_offsets[expert];
      rows = rs.expert_offsets[expert + 1] - row0;
    } else {
      row0 = rs.capacity + (expert - rs.E) * rs.T;
      rows = rs.T;
    }
  }
  return rows > 0;
}

// Token of an expert row, or -1 for a padding row.
__device__ __forceinline__ int row_token(const RowSpace &rs, int grow) {
  if (grow >= rs.capacity) return (grow - rs.capacity) % rs.T;
  const int p = rs.sorted_pairs[grow];
  return p >= rs.T * rs.k_max ? -1 : p / rs.k_max;
}

__device__ __forceinline__ bool row_real(const RowSpace &rs, int grow) {
  return grow >= rs.capacity || rs.sorted_pairs[grow] < rs.T * rs.k_max;
}

constexpr v8i kZero8 = {0, 0, 0, 0, 0, 0, 0, 0};

}  // namespace

// ------------------------------------------------------------------ gate/up
// h[row][o] = SiLU(g) * u with g = (G * sx[t]) * s_gate[o], u likewise, and
// G, U the e4m3 products accumulated in fp32 by the MFMA.
template <int MSUB>
__global__ __launch_bounds__(256) void gate_up_kernel(GemmArgs g) {
  const RowSpace &rs = g.rs;
  const int d = rs.d, f = rs.f;
  const int n_tiles = f >> 6;
  const int item_id = blockIdx.x / n_tiles;
  const int tile = blockIdx.x - item_id * n_tiles;
  int expert, row0, rows;
  if (!resolve_item(rs, item_id, expert, row0, rows)) return;
  const bool shared = expert >= rs.E;
  const size_t ex = (size_t)(shared ? expert - rs.E : expert);
  const uint8_t *wg = (shared ? g.w.ws_gate : g.w.w_gate) + ex * f * d;
  const uint8_t *wu = (shared ? g.w.ws_up : g.w.w_up) + ex * f * d;
  const float *sg = (shared ? g.w.ss_gate : g.w.s_gate) + ex * f;
  const float *su = (shared ? g.w.ss_up : g.w.s_up) + ex * f;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ln = lane & 15, kg = lane >> 4;
  const int o = (tile << 6) + (wave << 4) + ln;  // this lane's output channel
  const uint8_t *bgp = wg + (size_t)o * d + kg * 32;
  const uint8_t *bup = wu + (size_t)o * d + kg * 32;
  const int nk = (d + 127) >> 7;
  const bool half_tail = (d & 127) != 0;  // last K step holds 64 bytes: groups 2,3 idle
  const float sgo = sg[o], suo = su[o];

  for (int p0 = 0; p0 < rows; p0 += 16 * MSUB) {
    const int msub = min(MSUB, (rows - p0 + 15) >> 4);
    const uint8_t *ap[MSUB];
#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      const int r = p0 + m * 16 + ln;
      int tok = -1;
      if (m < msub && r < rows) tok = row_token(rs, row0 + r);
      ap[m] = tok >= 0 ? g.a + (size_t)tok * d + kg * 32 : nullptr;
    }
    v4f accg[MSUB], accu[MSUB];
#pragma unroll
    for (int m = 0; m < MSUB; ++m) accg[m] = accu[m] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int ks = 0; ks < nk; ++ks) {
      const int k = ks << 7;
      const bool kval = !(half_tail && ks == nk - 1 && kg >= 2);
      const v8i bg = kval ? load32(bgp + k) : kZero8;
      const v8i bu = kval ? load32(bup + k) : kZero8;
#pragma unroll
      for (int m = 0; m < MSUB; ++m) {
        if (m < msub) {
          const v8i av = (ap[m] && kval) ? load32(ap[m] + k) : kZero8;
          accg[m] = mfma_e4m3_16x16x128(av, bg, accg[m]);
          accu[m] = mfma_e4m3_16x16x128(av, bu, accu[m]);
        }
      }
    }

#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      if (m < msub) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = p0 + m * 16 + kg * 4 + i;
          if (r < rows) {
            const int grow = row0 + r;
            const int tok = row_token(rs, grow);
            float hv = 0.0f;
            if (tok >= 0) {
              const float sxt = g.a_scale[tok];
              const float gv = accg[m][i] * sxt * sgo;
              const float uv = accu[m][i] * sxt * suo;
              hv = gv / (1.0f + expf(-gv)) * uv;
            }
            g.out[(size_t)grow * f + o] = hv;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ requant
// One wave per real expert row: hq = e4m3(h * 448/amax), sh = amax/448.
__global__ __launch_bounds__(256) void requant_kernel(RowSpace rs, const float *__restrict__ h,
                                                      uint8_t *__restrict__ hq,
                                                      float *__restrict__ sh, int rows_total) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows_total || !row_real(rs, row)) return;
  quantize_row_wave(h + (size_t)row * rs.f, rs.f, hq + (size_t)row * rs.f, sh + row,
                    threadIdx.x & 63);
}

// ------------------------------------------------------------------ down
// y[row][c] = (Y * sh[row]) * s_down[c], Y = sum_o dec(hq[row][o]) dec(Wd[c][o]).
// F32A: y[row][c] = Y * s_down[c] with Y = sum_o h[row][o] dec(Wd[c][o]) on
// fp32 products (v_mfma_f32_16x16x4_f32; instruction i of a 128-wide step
// takes K index 32*(l/16) + i from lane l, for A and B alike).
constexpr int kDownSub = 2;  // 16-channel groups per wave -> 128 channels per workgroup

template <int MSUB, bool F32A>
__global__ __launch_bounds__(256) void down_kernel(GemmArgs g) {
  const RowSpace &rs = g.rs;
  const int d = rs.d, f = rs.f;
  const int n_tiles = (d + 127) >> 7;
  const int item_id = blockIdx.x / n_tiles;
  const int tile = blockIdx.x - item_id * n_tiles;
  int expert, row0, rows;
  if (!resolve_item(rs, item_id, expert, row0, rows)) return;
  const bool shared = expert >= rs.E;
  const size_t ex = (size_t)(shared ? expert - rs.E : expert);
  const uint8_t *wd = (shared ? g.w.ws_down : g.w.w_down) + ex * d * f;
  const float *sd = (shared ? g.w.ss_down : g.w.s_down) + ex * d;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ln = lane & 15, kg = lane >> 4;
  int oc[kDownSub];
  const uint8_t *bp[kDownSub];
#pragma unroll
  for (int n = 0; n < kDownSub; ++n) {
    oc[n] = (tile << 7) + (wave << 5) + (n << 4) + ln;
    bp[n] = oc[n] < d ? wd + (size_t)oc[n] * f + kg * 32 : nullptr;
  }
  const int nk = (f + 127) >> 7;
  const bool half_tail = (f & 127) != 0;

  for (int p0 = 0; p0 < rows; p0 += 16 * MSUB) {
    const int msub = min(MSUB, (rows - p0 + 15) >> 4);
    size_t aoff[MSUB];
    bool aok[MSUB];
#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      const int r = p0 + m * 16 + ln;
      aok[m] = m < msub && r < rows && row_real(rs, row0 + r);
      aoff[m] = (size_t)(row0 + r) * f + kg * 32;
    }
    v4f acc[MSUB][kDownSub];
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int n = 0; n < kDownSub; ++n) acc[m][n] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int ks = 0; ks < nk; ++ks) {
      const int k = ks << 7;
      const bool kval = !(half_tail && ks == nk - 1 && kg >= 2);
      v8i b[kDownSub];
#pragma unroll
      for (int n = 0; n < kDownSub; ++n) b[n] = (kval && bp[n]) ? load32(bp[n] + k) : kZero8;
#pragma unroll
      for (int m = 0; m < MSUB; ++m) {
        if (m < msub) {
          if constexpr (!F32A) {
            const v8i av = (aok[m] && kval) ? load32(g.a + aoff[m] + k) : kZero8;
#pragma unroll
            for (int n = 0; n < kDownSub; ++n) acc[m][n] = mfma_e4m3_16x16x128(av, b[n], acc[m][n]);
          } else {
            float af[32];
            const float *src = g.a32 + aoff[m] + k;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              v4f v = (aok[m] && kval) ? *reinterpret_cast<const v4f *>(src + 4 * q)
                                       : v4f{0.f, 0.f, 0.f, 0.f};
              af[4 * q] = v.x;
              af[4 * q + 1] = v.y;
              af[4 * q + 2] = v.z;
              af[4 * q + 3] = v.w;
            }
#pragma unroll
            for (int n = 0; n < kDownSub; ++n) {
#pragma unroll
              for (int q = 0; q < 8; ++q) {
                const uint32_t wword = (uint32_t)b[n][q];
                const v2f lo = e4m3x2_to_f32<false>(wword);
                const v2f hi = e4m3x2_to_f32<true>(wword);
                acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[4 * q], lo.x, acc[m][n], 0, 0, 0);
                acc[m][n] =
                    __builtin_amdgcn_mfma_f32_16x16x4f32(af[4 * q + 1], lo.y, acc[m][n], 0, 0, 0);
                acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[4 * q + 2], hi.x, acc[m][n], 0, 0, 0);
                acc[m][n] =
                    __builtin_amdgcn_mfma_f32_16x16x4f32(af[4 * q + 3], hi.y, acc[m][n], 0, 0, 0);
              }
            }
          }
        }
      }
    }

#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      if (m < msub) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = p0 + m * 16 + kg * 4 + i;
          if (r < rows) {
            const int grow = row0 + r;
            const bool real = row_real(rs, grow);
            const float shr = (!F32A && real) ? g.a_scale[grow] : 1.0f;
#pragma unroll
            for (int n = 0; n < kDownSub; ++n) {
              if (oc[n] < d) {
                float yv = 0.0f;
                if (real) yv = F32A ? acc[m][n][i] * sd[oc[n]] : acc[m][n][i] * shr * sd[oc[n]];
                g.out[(size_t)grow * d + oc[n]] = yv;
              }
            }
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ combine
// out[t] = sum_j w[t,j] * y[inv[t,j]] over valid slots in order, then + the
// shared experts' rows in order.  One workgroup per token, 4 columns a lane.
__global__ __launch_bounds__(256) void combine_kernel(RowSpace rs, const float *__restrict__ y,
                                                      const int32_t *__restrict__ ids,
                                                      const float *__restrict__ w,
                                                      const int32_t *__restrict__ inv,
                                                      float *__restrict__ out) {
  const int t = blockIdx.x;
  const int d = rs.d, K = rs.k_max;
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < K; ++j) {
      const int p = t * K + j;
      if (ids[p] < 0) continue;
      const float wj = w[p];
      const v4f v = *reinterpret_cast<const v4f *>(y + (size_t)inv[p] * d + c);
      acc += wj * v;
    }
    for (int s = 0; s < rs.S; ++s) {
      const v4f v =
          *reinterpret_cast<const v4f *>(y + ((size_t)rs.capacity + (size_t)s * rs.T + t) * d + c);
      acc += v;
    }
    *reinterpret_cast<v4f *>(out + (size_t)t * d + c) = acc;
  }
}

// ------------------------------------------------------------------ launchers

static int grid_items(const RowSpace &rs) { return rs.items ? rs.max_items : rs.E + rs.S; }

hipError_t launch_gate_up(const RowSpace &rs, const uint8_t *xq, const float *sx,
                          const ExpertWeights &w, float *h, int32_t msub, hipStream_t stream) {
  GemmArgs g{rs, xq, sx, nullptr, w, h};
  const int blocks = grid_items(rs) * (rs.f >> 6);
  if (blocks == 0) return hipSuccess;
  if (msub >= 8)
    gate_up_kernel<8><<<blocks, 256, 0, stream>>>(g);
  else if (msub >= 4)
    gate_up_kernel<4><<<blocks, 256, 0, stream>>>(g);
  else if (msub >= 2)
    gate_up_kernel<2><<<blocks, 256, 0, stream>>>(g);
  else
    gate_up_kernel<1><<<blocks, 256, 0, stream>>>(g);
  return hipGetLastError();
}

hipError_t launch_requant(const RowSpace &rs, const float *h, uint8_t *hq, float *sh,
                          hipStream_t stream) {
  const int rows_total = rs.capacity + rs.S * rs.T;
  if (rows_total == 0) return hipSuccess;
  requant_kernel<<<(rows_total + 3) / 4, 256, 0, stream>>>(rs, h, hq, sh, rows_total);
  return hipGetLastError();
}

hipError_t launch_down(const RowSpace &rs, const uint8_t *hq, const float *sh, const float *h32,
                       const ExpertWeights &w, float *y, int32_t msub, hipStream_t stream) {
  GemmArgs g{rs, hq, sh, h32, w, y};
  const int blocks = grid_items(rs) * ((rs.d + 127) >> 7);
  if (blocks == 0) return hipSuccess;
  if (h32) {
    down_kernel<1, true><<<blocks, 256, 0, stream>>>(g);
  } else if (msub >= 8) {
    down_kernel<8, false><<<blocks, 256, 0, stream>>>(g);
  } else if (msub >= 4) {
    down_kernel<4, false><<<blocks, 256, 0, stream>>>(g);
  } else if (msub >= 2) {
    down_kernel<2, false><<<blocks, 256, 0, stream>>>(g);
  } else {
    down_kernel<1, false><<<blocks, 256, 0, stream>>>(g);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const RowSpace &rs, const float *y, const int32_t *ids, const float *w,
                          const int32_t *inv_pairs, float *out, hipStream_t stream) {
  if (rs.T == 0) return hipSuccess;
  combine_kernel<<<rs.T, 256, 0, stream>>>(rs, y, ids, w, inv_pairs, out);
  return hipGetLastError();
}

}  // namespace fp8moe
