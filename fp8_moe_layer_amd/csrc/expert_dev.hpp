// expert_dev.hpp -- device functions of the expert FFN stages of the W8A8 FP8 MoE layer on gfx950:
// gate/up grouped GEMM with the SiLU*up epilogue, per-row e4m3
// requantisation, down-projection grouped GEMM, and the weighted combine.
//
// "Routage MoE entre GPU": each expert is a feed-forward network with its
// own weights and only the selected experts process a token; the outputs are
// weighted, summed and put back in token order.  W8A8 FP8: Alpha-MoE article,
// opening section.
//
// Grouped GEMM schedule: weight-stationary, one workgroup per (work item,
// tile of output channels[, K split]).  A work item is an expert and up to
// 16*MSUB of its rows (16*ML with the two-shape kernel), so a decode-sized
// batch puts all of an expert's rows in one item and each active expert's
// weights cross HBM exactly once.
//
// Workgroup = W compute waves (1..8, chosen by the host) + 1 loader wave
// (2 for 256-row passes):
//  - the loader gathers the item's activation rows (e4m3) into a ring of four
//    LDS chunks with global_load_lds_dwordx4, three chunks ahead of the
//    compute waves (exact vmcnt waits, so only the chunk due next is waited
//    for), after one batch of row lookups; the rows' activation scales go to
//    an LDS table by direct-to-LDS dword loads issued ahead of the first
//    chunk;
//  - each compute wave streams NB weight operands of 16 rows (gate and up
//    rows of 16 channels, or 32 down channels) from HBM into registers
//    through a PF-deep prefetch ring, reads the activation fragments from LDS
//    (four row groups at a time) and runs v_mfma_f32_16x16x128_f8f6f4;
//  - one s_barrier per chunk hands buffers between them.  The compute side
//    waits only on LDS counters, so its weight prefetches stay in flight
//    across it.
//
// MFMA operand layout (same for A = activation rows and B = weight rows):
// lane l holds row l%16 and, of each 128-byte K step, the bytes
// [16*(l/16), +16) and [64 + 16*(l/16), +16).  The weights are stored in
// that order (tile order, moe_weights), so each weight piece load of a wave
// is 1 KB contiguous; an activation piece load covers 16 rows x 64 bytes.
// Result tile: lane l, element i = C[4*(l/16) + i][l%16].
#pragma once
#include "common.hpp"
#include "internal.hpp"

namespace fp8moe {



struct GemmArgs {
  RowSpace rs;
  const uint8_t *a;      // gate/up: xq [T][d]; down: hq [rows][f]
  const float *a_scale;  // sx [T] or sh [rows]
  const float *a32;      // down, fp32 mode: h [rows][f]
  ExpertWeights w;
  float *out;            // h [rows][f] or y [splits][rows][d]
  int32_t splits;        // K splits (down only; partial sums go to separate y slabs)
  int32_t ksplit;        // bytes of K per split (multiple of the chunk size)
  // Down projection: when set, y is written here in fp16 (same layout; values
  // beyond +-65504 saturate) instead of fp32 to `out`.
  _Float16 *out16 = nullptr;
  // A-resident tiles (ares_tile): consecutive N-tiles per workgroup.
  int32_t ntg = 1;
  // Decode down projection: tile t of expert e starts its K loop at step
  // ((t + 5e) * krot) % nks and wraps (0: no rotation).  When all of a
  // launch's workgroups run in one round they otherwise walk their weight
  // rows in step, every one at the same K offset at the same time.
  int32_t krot = 0;
  // Gate/up with the requantisation fused into its epilogue (the tile spans
  // all of f): hq [rows][f] e4m3 codes and hsc [rows] = amax/448 instead of h.
  uint8_t *hq = nullptr;
  float *hsc = nullptr;
};

// real: the item's rows that hold pairs (the rest of its rows are segment
// padding, whose h and y no stage reads: the epilogues skip their stores);
// without a work list every row counts as real.
__device__ __forceinline__ bool resolve_item(const RowSpace &rs, int item_id, int &expert,
                                             int &row0, int &rows, int &real) {
  if (rs.items) {
    if (item_id >= *rs.n_items) return false;
    const WorkItem it = rs.items[item_id];
    expert = it.expert;
    row0 = it.row0;
    rows = it.rows;
    real = min(max(it.real, 0), rows);
    // an item lies inside its expert's rows (routed: [0, capacity); shared
    // expert s: [capacity + s*T, +T))
    if constexpr (kDebugChecks) {
      const bool in = expert >= 0 && expert < rs.E + rs.S && row0 >= 0 && rows >= 0 &&
                      (expert < rs.E ? row0 + rows <= rs.capacity
                                     : row0 >= rs.capacity + (expert - rs.E) * rs.T &&
                                           row0 + rows <= rs.capacity + (expert - rs.E + 1) * rs.T);
      if (!dcheck(in, kDbgPermute)) return false;
    }
  } else {
    expert = item_id;
    if (expert < rs.E) {
      row0 = rs.expert_offsets[expert];
      rows = rs.expert_offsets[expert + 1] - row0;
    } else {
      row0 = rs.capacity + (expert - rs.E) * rs.T;
      rows = rs.T;
    }
    real = rows;
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
  if (grow >= rs.capacity) return true;
  const int sp = rs.sorted_pairs[grow];
  // a pair index or the padding sentinel T*k_max (checked in the debug build)
  if constexpr (kDebugChecks)
    if (!dcheck(sp >= 0 && sp <= rs.T * rs.k_max, kDbgRow)) return false;
  return sp < rs.T * rs.k_max;
}

// Activation row read for expert row `grow` of a GEMM (the token for gate/up,
// the expert row itself for down), or -1 for a padding row or !ok.  sp is
// sorted_pairs[min(grow, capacity - 1)], loaded by the caller.  Branch-free,
// so that the caller's loads are not sunk into branches and stay together.
template <bool GATEUP>
__device__ __forceinline__ int act_row(const RowSpace &rs, int grow, int sp, bool ok) {
  const bool sh_row = grow >= rs.capacity;
  bool real = sh_row | (sp < rs.T * rs.k_max);
  // sp: a pair index or the padding sentinel T*k_max (checked in the debug build)
  if constexpr (kDebugChecks) real = real && (sh_row || dcheck(sp >= 0 && sp <= rs.T * rs.k_max, kDbgRow));
  int a = grow;
  if (GATEUP) a = sh_row ? (grow - rs.capacity) % rs.T : sp / rs.k_max;
  return (ok & real) ? a : -1;
}

// LDS-only workgroup barrier: waits for this wave's LDS operations, not for
// its outstanding global loads.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
// Loader side: its direct-to-LDS loads are counted by vmcnt.
__device__ __forceinline__ void barrier_after_loads() {
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) void *lds_ptr;

// 64 zero bytes: the source of activation pieces for padding rows and K
// past the end.  Never written (each translation unit has its own copy).
static __device__ __attribute__((aligned(64))) uint8_t g_zero_piece[64];

// Weight operands of one compute wave.  Operand nb holds the weight rows of
// output channel ch[nb] (gate, up, gate, ... for gate/up; down channels
// otherwise), read as MFMA B operands; wsc[nb] is that channel's weight
// scale, loaded at set-up so the epilogue waits on no global load.  A lane
// past the last channel (partial last tile) reads valid rows and stores
// nothing.
template <int NB, bool GATEUP, bool NT>
struct WOperands {
  // bw: the 2 KB weight tile of the split's first K step for channel group
  // nb (the same for the whole wave, so it can live in scalar registers);
  // lane l reads its 16 bytes at l * 16 and 1024 + l * 16 of each tile.
  const uint8_t *bw[NB];
  int l16;
  int ch[NB];
  float wsc[NB];
  int nks;      // K steps of this split
  int rot = 0;  // logical step ks < nks reads physical step (ks + rot) % nks

  // c0: the wave's first output channel; k_begin: first K byte of the split.
  __device__ __forceinline__ void init(const GemmArgs &g, bool shared, size_t ex, int c0, int k_begin,
                                       int nks_, int lane) {
    const int N = GATEUP ? g.rs.f : g.rs.d;
    const int K = GATEUP ? g.rs.d : g.rs.f;
    const int KT = (K + 127) >> 7;  // weight tiles along K
    nks = nks_;
    l16 = lane * 16;
    if constexpr (kDebugChecks) dcheck((c0 & 15) == 0, kDbgTile);  // the group clamp below
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int o;
      const uint8_t *wbase;
      const float *sbase;
      if (GATEUP) {
        o = c0 + (nb >> 1) * 16 + (lane & 15);
        wbase = ((nb & 1) == 0 ? (shared ? g.w.ws_gate : g.w.w_gate) : (shared ? g.w.ws_up : g.w.w_up)) +
                ex * (size_t)N * KT * 128;
        sbase = (nb & 1) == 0 ? (shared ? g.w.ss_gate : g.w.s_gate) : (shared ? g.w.ss_up : g.w.s_up);
      } else {
        o = c0 + nb * 16 + (lane & 15);
        wbase = (shared ? g.w.ws_down : g.w.w_down) + ex * (size_t)N * KT * 128;
        sbase = shared ? g.w.ss_down : g.w.s_down;
      }
      const int orow = o < N ? o : N - 1;
      ch[nb] = o;
      wsc[nb] = sbase[ex * N + orow];
      // tile order: 16 rows x 128 K bytes per 2 KB tile.  c0 is a multiple of
      // 16 and so is N: a group of 16 channels past N clamps, as a whole, to
      // the last group (the rows of channel N - 1, as orow)
      const int grp = min((c0 >> 4) + (GATEUP ? (nb >> 1) : nb), (N >> 4) - 1);
      bw[nb] = wbase + ((size_t)grp * KT + (k_begin >> 7)) * 2048;
    }
  }

  // Weight tile of K step ks: two contiguous 1 KB halves.  Past the end the
  // step is clamped to the last one (its activation pieces are zero); the
  // zero padding of a 64-byte tail step meets zero activation pieces.
  __device__ __forceinline__ void load(v8i (&b)[NB], int ks) const {
    ks = ks < nks ? (ks + rot >= nks ? ks + rot - nks : ks + rot) : nks - 1;
    const int o0 = ks * 2048 + l16;
    const int o1 = o0 + 1024;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const v4i lo = NT ? load16_nt(bw[nb] + o0) : load16(bw[nb] + o0);
      const v4i hi = NT ? load16_nt(bw[nb] + o1) : load16(bw[nb] + o1);
      b[nb] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  }
};

// Epilogue of one row pass (rows p0 .. p0+prow-1 of the item starting at
// expert row row0): gate/up writes h = SiLU(g)*u, the down projection its
// split's y slab.  rsc: the pass's activation scale per row (0 for a
// padding row) in LDS.
// e^(-g) for the SiLU in a few instructions: 2^y with y = -g*log2(e)
// rounded to fp32, times 2^r ~ 1 + r*ln 2 for the residual r (the product's
// rounding error, recovered by an fma, plus the part of log2(e) below fp32),
// so the result stays within a few ulp over the whole range.  v_exp_f32
// gives +inf past 2^128 (the SiLU then gives 0) and 0 below the fp32 range
// (SiLU(g) = g).
__device__ __forceinline__ float exp_neg(float g) {
  constexpr float kLog2e = 1.44269502f;       // log2(e) rounded to fp32
  constexpr float kLog2eLo = 1.92596299e-8f;  // log2(e) - kLog2e
  constexpr float kLn2 = 0.693147181f;
  const float y = -g * kLog2e;
  const float r = fmaf(-g, kLog2e, -y) + (-g) * kLog2eLo;
  return __builtin_amdgcn_exp2f(y) * (1.0f + r * kLn2);
}

// O16 (down projection): 1 writes y in fp16 (g.out16), 0 in fp32 (g.out), -1
// decides at run time by whether g.out16 is set (a kernel that knows which
// lets the compiler drop the other path's registers).
template <int MSUB, int NB, bool GATEUP, bool NT, int O16 = -1>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs &g, const v4f (&acc)[MSUB][NB],
                                              const WOperands<NB, GATEUP, NT> &wo, const float *rsc,
                                              int row0, int p0, int prow, int msub, int split,
                                              int lane) {
  const RowSpace &rs = g.rs;
  const int N = GATEUP ? rs.f : rs.d;
  const int kg = lane >> 4;
  // Lane (ln, kg) holds rows m*16 + kg*4 + i of channel wo.ch[nb].  prow and
  // msub here count the pass's rows to store: the rows that hold pairs (an
  // expert segment's padding rows follow its last pair, and no stage reads
  // their h or y), so only the last stored row group is masked (a pass of
  // 16*MSUB stored rows takes the unmasked path).  The store address
  // advances by one row per element (no table of row offsets).  Stores are
  // non-temporal: the output stream does not push the weight stream's
  // neighbours (activation rows, tables) out of L2.
  const bool full = prow == 16 * MSUB;
  const bool to16 = O16 == 1 || (O16 < 0 && g.out16 != nullptr);
  if (GATEUP) {
#pragma unroll
    for (int cg = 0; cg < NB / 2; ++cg) {
      if (wo.ch[2 * cg] >= N) continue;
      const float sgo = wo.wsc[2 * cg], suo = wo.wsc[2 * cg + 1];
      float *hp = g.out + (size_t)(row0 + p0 + kg * 4) * N + wo.ch[2 * cg];
      auto h_of = [&](int m, int i, float sxr) {
        const float gv = acc[m][2 * cg][i] * sxr * sgo;
        const float uv = acc[m][2 * cg + 1][i] * sxr * suo;
        // SiLU(g)*u with the reciprocal instruction (1 ulp) for the divide
        return gv * __builtin_amdgcn_rcpf(1.0f + exp_neg(gv)) * uv;
      };
      if (full) {
#pragma unroll
        for (int m = 0; m < MSUB; ++m) {
          const v4f sx4 = *reinterpret_cast<const v4f *>(rsc + m * 16 + kg * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            __builtin_nontemporal_store(h_of(m, i, sx4[i]), hp);
            hp += i < 3 ? N : 13 * N;
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < MSUB; ++m) {
          if (m < msub) {
            const v4f sx4 = *reinterpret_cast<const v4f *>(rsc + m * 16 + kg * 4);
            const int rlim = prow - (m * 16 + kg * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float hv = h_of(m, i, sx4[i]);
              if (m < msub - 1 || i < rlim) __builtin_nontemporal_store(hv, hp);
              hp += i < 3 ? N : 13 * N;
            }
          }
        }
      }
    }
  } else {
    const size_t yoff = (size_t)split * (rs.capacity + rs.S * rs.T) * N + (size_t)(row0 + p0 + kg * 4) * N;
    if (to16) {
      // fp16 y: lanes ln and ln^1 hold channels c, c+1 of a row; the even lane
      // stores both as one 32-bit word (the odd lane's value comes over DPP,
      // in every lane before any store condition).  A wave covers 64 bytes of
      // a row, half a cache line: ordinary stores, so L2 merges the two
      // halves before they go to memory.
      _Float16 *yh = g.out16 + yoff;
      const bool even = (lane & 1) == 0;
      const bool live_nt = __builtin_amdgcn_ballot_w64(wo.ch[NB - 1] >= N) == 0;
      size_t yrow = 0;
#pragma unroll
      for (int m = 0; m < MSUB; ++m) {
        if (m < msub) {
          const v4f sh4 = *reinterpret_cast<const v4f *>(rsc + m * 16 + kg * 4);
          const int rlim = full ? 4 : prow - (m * 16 + kg * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const float v = fminf(fmaxf(acc[m][nb][i] * sh4[i] * wo.wsc[nb], -65504.0f), 65504.0f);
              const float u = dpp_mov<kDppQuadXor1>(v);
              if (even && (m < msub - 1 || i < rlim) && (live_nt || wo.ch[nb] < N)) {
                const v2h pk = {(_Float16)v, (_Float16)u};
                *reinterpret_cast<v2h *>(yh + yrow + wo.ch[nb]) = pk;
              }
            }
            yrow += i < 3 ? N : 13 * N;
          }
        }
      }
      return;
    }
    float *yp = g.out + yoff;
    // one y element (non-temporal: a wave covers a whole 128-byte line of a row)
    auto put = [&](float v, size_t at) { __builtin_nontemporal_store(v, yp + at); };
    size_t yrow = 0;  // offset of the current row from yp
    // every lane's channels inside N (all but a partial last tile): no
    // per-store channel mask
    const bool live = __builtin_amdgcn_ballot_w64(wo.ch[NB - 1] >= N) == 0;
    if (full && live) {
#pragma unroll
      for (int m = 0; m < MSUB; ++m) {
        const v4f sh4 = *reinterpret_cast<const v4f *>(rsc + m * 16 + kg * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) put(acc[m][nb][i] * sh4[i] * wo.wsc[nb], yrow + wo.ch[nb]);
          yrow += i < 3 ? N : 13 * N;
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < MSUB; ++m) {
        if (m < msub) {
          const v4f sh4 = *reinterpret_cast<const v4f *>(rsc + m * 16 + kg * 4);
          const int rlim = prow - (m * 16 + kg * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if (m < msub - 1 || i < rlim) {
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                if (wo.ch[nb] < N) put(acc[m][nb][i] * sh4[i] * wo.wsc[nb], yrow + wo.ch[nb]);
            }
            yrow += i < 3 ? N : 13 * N;
          }
        }
      }
    }
  }
}

// Gate/up epilogue with the per-row requantisation fused in, for a tile that
// spans all f channels of its rows (W waves of NB/2 channel groups each, the
// item's rows in one pass).  h = SiLU(g)*u exactly as the h epilogue forms it;
// each wave's row maxima of |h| over its channels (lanes of one DPP row hold
// one row's 16 channels of a group) go to LDS, pmax[wave][row]; after one
// workgroup barrier (the loader wave takes it too) a row's amax is the
// maximum over the waves, and hq = e4m3(h * (448/amax)), hsc = amax/448 --
// the separate requantisation's operations on the same h, so the same codes
// and scales bit for bit, with no fp32 h in memory.  prow and msub count the
// rows to store (those that hold pairs): the down projection gives segment
// padding rows zero activations and scale 0 without reading hq or hsc.
template <int MSUB, int NB, bool NT>
__device__ __forceinline__ void gemm_epilogue_rq(const GemmArgs &g, const v4f (&acc)[MSUB][NB],
                                                 const WOperands<NB, true, NT> &wo,
                                                 const float *rsc, float *pmax, int row0, int p0,
                                                 int prow, int msub, int lane, int wave, int W) {
  constexpr int MP = 16 * MSUB;
  const int N = g.rs.f;
  // the row offsets below are formed here, not hoisted above the K loop
  // (where they would be held in registers the loop needs)
  asm volatile("" : "+v"(lane));
  const int kg = lane >> 4, ln = lane & 15;
  // h of (row group m, element i, channel group cg), formed from the
  // accumulators both times it is needed (the same operations, so the same
  // bits): holding it across the barrier would cost registers the K loop uses
  auto h_of = [&](int m, int cg, int i, float sxr) {
    const float gv = acc[m][2 * cg][i] * sxr * wo.wsc[2 * cg];
    const float uv = acc[m][2 * cg + 1][i] * sxr * wo.wsc[2 * cg + 1];
    return gv * __builtin_amdgcn_rcpf(1.0f + exp_neg(gv)) * uv;
  };
#pragma unroll
  for (int m = 0; m < MSUB; ++m) {
    const v4f sx4 = *reinterpret_cast<const v4f *>(rsc + m * 16 + kg * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float pm = 0.0f;
#pragma unroll
      for (int cg = 0; cg < NB / 2; ++cg)
        if (wo.ch[2 * cg] < N) pm = fmaxf(pm, fabsf(h_of(m, cg, i, sx4[i])));
      // the row's maximum over the 16 lanes of this DPP row
      pm = fmaxf(pm, dpp_mov<kDppQuadXor1>(pm));
      pm = fmaxf(pm, dpp_mov<kDppQuadXor2>(pm));
      pm = fmaxf(pm, dpp_mov<kDppHalfMirror>(pm));
      pm = fmaxf(pm, dpp_mov<kDppMirror>(pm));
      if (ln == 0) pmax[wave * MP + m * 16 + kg * 4 + i] = pm;
    }
    // one row group at a time: interleaving the groups' SiLU chains would
    // raise register pressure past the K loop's
    __builtin_amdgcn_sched_barrier(0);
  }
  barrier_lds();
  const bool full = prow == MP;
#pragma unroll
  for (int m = 0; m < MSUB; ++m) {
    if (m < msub) {
      const v4f sx4 = *reinterpret_cast<const v4f *>(rsc + m * 16 + kg * 4);
      const int rlim = full ? 4 : prow - (m * 16 + kg * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = m * 16 + kg * 4 + i;
        if (m < msub - 1 || i < rlim) {
          float amax = pmax[r];
          for (int w = 1; w < W; ++w) amax = fmaxf(amax, pmax[w * MP + r]);
          float rq = 1.0f, sq = 1.0f;
          if (amax != 0.0f) {
            rq = kE4m3Max / amax;
            sq = amax / kE4m3Max;
          }
          uint8_t *q = g.hq + (size_t)(row0 + p0 + r) * N;
#pragma unroll
          for (int cg = 0; cg < NB / 2; ++cg) {
            if (wo.ch[2 * cg] < N) {
              const float hv = h_of(m, cg, i, sx4[i]);
              if constexpr (kDebugChecks) dcheck(__builtin_isfinite(hv), kDbgNonFinite);
              q[wo.ch[2 * cg]] = (uint8_t)(e4m3x4(hv * rq, 0.0f, 0.0f, 0.0f) & 0xffu);
            }
          }
          if (wave == 0 && ln == 0) g.hsc[row0 + p0 + r] = sq;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------------------------------------ grouped GEMM

template <int MSUB>
struct Chunk {
  static constexpr int MP = 16 * MSUB;                 // rows per pass
  static constexpr int KSC = MSUB >= 8 ? 1 : 8 / MSUB; // K steps per chunk
  static constexpr int BYTES = MSUB * KSC * 2048;      // 16 KB (32 KB for 256-row passes)
  static constexpr int NBUF = 4;                       // LDS ring; loads run NBUF-1 chunks ahead
  static constexpr int LOADERS = MSUB > 8 ? 2 : 1;     // loader waves, 16 loads per chunk each
  static constexpr int LPC = MSUB * KSC * 2 / LOADERS; // direct-to-LDS loads per chunk and loader
  static constexpr int MPL = MSUB / LOADERS;           // row groups per loader wave
  // weight prefetch depth in k steps (registers allow 4 when few row tiles)
  static constexpr int PF = MSUB <= 2 ? 4 : 2;
  // LDS: the activation ring, then a table of the activation scale of each
  // row of the current pass (two copies by pass parity), 0 for a padding
  // row.  The compute waves fill it while their first weight loads are in
  // flight, so the epilogue needs no global loads on its critical path.
  static constexpr int RING = NBUF * BYTES;
  static constexpr int LDS = RING + 2 * MP * (int)sizeof(float);
  // with the fused requantisation: + the waves' row maxima (pmax[wave][row],
  // up to 12 waves)
  static constexpr int LDS_RQ = LDS + 12 * MP * (int)sizeof(float);
};

// LDS of the persistent kernel's GEMM phases (row passes of up to 128 rows).
constexpr int kGemmLdsBytes = Chunk<8>::LDS;

// K granule of a split: whole chunks.
__host__ __device__ constexpr int split_granule(int msub) {
  return 128 * (msub >= 8 ? 1 : 8 / msub);
}

// s_waitcnt vmcnt(n * 16): n chunks of loads may stay in flight.
__device__ __forceinline__ void loader_wait_barrier(int chunks_in_flight) {
  if (chunks_in_flight >= 2)
    asm volatile("s_waitcnt vmcnt(32)\n\ts_barrier" ::: "memory");
  else if (chunks_in_flight == 1)
    asm volatile("s_waitcnt vmcnt(16)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

// GATEUP: out = h[rows][f]; a wave holds NB/2 channel groups of 16, each as
//         a (gate rows, up rows) pair of weight operands.
// else:   out = y[split][rows][d]; NB channel groups of 16 per wave.
// One call computes tile `bid` (= (item * n_tiles + tile) * splits + split)
// with a workgroup of W = blockDim.x/64 - LOADERS compute waves followed by
// the loader wave(s); the tile is W * (GATEUP ? 8 : 16) * NB output channels
// wide.  abuf: Chunk<MSUB>::LDS bytes of LDS, 1024-byte aligned.  Returns
// early (uniformly) for an empty item.
// NT: the weight loads carry the non-temporal hint, so that a weight stream
// read once does not push the activation rows and row tables out of L2.
// RQ (gate/up, the tile spanning all f): the requantisation is fused into
// the epilogue (gemm_epilogue_rq); abuf then holds Chunk<MSUB>::LDS_RQ bytes
// and every wave, the loader included, takes one more barrier per pass.
template <int MSUB, int NB, bool GATEUP, bool NT = false, bool RQ = false>
__device__ __forceinline__ void wsgemm_tile(const GemmArgs &g, int bid, uint8_t *abuf) {
  using C = Chunk<MSUB>;
  static_assert(C::LPC == 16 && C::NBUF == 4, "loader_wait_barrier assumes 16 loads per chunk");
  const int W = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6) - C::LOADERS);  // compute waves

  const RowSpace &rs = g.rs;
  const int K = GATEUP ? rs.d : rs.f;
  const int N = GATEUP ? rs.f : rs.d;
  static_assert(!GATEUP || NB % 2 == 0, "gate/up operands come in pairs");
  constexpr int CH_WAVE = GATEUP ? 8 * NB : 16 * NB;
  const int CH_WG = W * CH_WAVE;
  const int n_tiles = (N + CH_WG - 1) / CH_WG;
  const int split = bid % g.splits;
  bid /= g.splits;
  const int tile = bid % n_tiles;
  const int item_id = bid / n_tiles;
  int expert, row0, rows, real;
  if (!resolve_item(rs, item_id, expert, row0, rows, real)) return;
  const int k_begin = split * g.ksplit;
  const int k_end = min(K, k_begin + g.ksplit);
  if (k_begin >= k_end) return;
  const int nks = (k_end - k_begin + 127) >> 7;         // K steps in this split
  // K steps are processed PF at a time; steps past nks multiply zero
  // activation pieces by a repeat of the last weight step.
  const int nks_pf = (nks + C::PF - 1) / C::PF * C::PF;
  const int nchunks = (nks_pf + C::KSC - 1) / C::KSC;  // LDS chunks of KSC steps
  const int krot = (!GATEUP && g.krot && nks > 1) ? ((tile + 5 * expert) * g.krot) % nks : 0;

  const bool shared = expert >= rs.E;
  const size_t ex = (size_t)(shared ? expert - rs.E : expert);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, kg = lane >> 4;

  float *row_scale = reinterpret_cast<float *>(abuf + C::RING);

  if (wave >= W) {
    // ---------------- loader waves: activation rows -> LDS, chunk by chunk;
    // loader j gathers row groups [j*MPL, (j+1)*MPL)
    const int mbase = (wave - W) * C::MPL;
    const uint8_t *abase[C::MPL];
    int pass = 0;
    for (int p0 = 0; p0 < rows; p0 += C::MP, ++pass) {
      const int prow = min(C::MP, rows - p0);
      const int msub = (prow + 15) >> 4;
      // The row lookups of all the loader's row groups, and of its share of
      // the pass's scale table (rows tfirst + 64*t + lane of the pass), are
      // issued together (unconditional loads at clamped indices), so a
      // pass's gather starts after one memory latency, not one or two per
      // row group.
      constexpr int TB = (C::MP / kWave + C::LOADERS - 1) / C::LOADERS;
      constexpr int TBn = TB > 0 ? TB : 1;  // table blocks of 64 rows per loader
      const int tfirst = (wave - W) * TBn * kWave;
      int grow[C::MPL], sp[C::MPL], tgrow[TBn], tsp[TBn];
#pragma unroll
      for (int mm = 0; mm < C::MPL; ++mm) {
        grow[mm] = row0 + min(p0 + (mbase + mm) * 16 + ln, rows - 1);
        sp[mm] = rs.sorted_pairs[min(grow[mm], rs.capacity - 1)];
      }
#pragma unroll
      for (int t = 0; t < TBn; ++t) {
        tgrow[t] = row0 + min(p0 + tfirst + t * kWave + lane, rows - 1);
        tsp[t] = rs.sorted_pairs[min(tgrow[t], rs.capacity - 1)];
      }
#pragma unroll
      for (int mm = 0; mm < C::MPL; ++mm) {
        const int r = p0 + (mbase + mm) * 16 + ln;
        const int a = act_row<GATEUP>(rs, grow[mm], sp[mm], mbase + mm < msub && r < rows);
        abase[mm] = a < 0 ? nullptr : g.a + (size_t)a * K;
      }
      const float *tsrc[TBn];
#pragma unroll
      for (int t = 0; t < TBn; ++t) {
        const int a = act_row<GATEUP>(rs, tgrow[t], tsp[t], tfirst + t * kWave + lane < prow);
        tsrc[t] = a < 0 ? reinterpret_cast<const float *>(g_zero_piece) : g.a_scale + a;
      }
      // The table goes to LDS by direct-to-LDS dword loads (a padding row
      // loads a zero) issued before chunk 0's, so the wait for chunk 0 also
      // covers them; lanes past the table stay idle.
      float *rsc = row_scale + (pass & 1) * C::MP;
#pragma unroll
      for (int t = 0; t < TBn; ++t)
        if (tfirst + t * kWave + lane < C::MP)
          __builtin_amdgcn_global_load_lds(tsrc[t], (lds_ptr)(rsc + tfirst + t * kWave), 4, 0, 0);
      auto issue = [&](int c) {
        uint8_t *dst = abuf + (c % C::NBUF) * C::BYTES;
#pragma unroll
        for (int mm = 0; mm < C::MPL; ++mm) {
          const int m = mbase + mm;
#pragma unroll
          for (int s = 0; s < C::KSC; ++s) {
#pragma unroll
            for (int p = 0; p < 2; ++p) {
              const int lks = c * C::KSC + s;  // logical step; past nks: zeros
              const int pks = lks + krot >= nks ? lks + krot - nks : lks + krot;
              const int kb = k_begin + pks * 128 + p * 64 + kg * 16;
              const uint8_t *src = (abase[mm] && lks < nks && kb < k_end) ? abase[mm] + kb : g_zero_piece;
              __builtin_amdgcn_global_load_lds(src, (lds_ptr)(dst + ((m * C::KSC + s) * 2 + p) * 1024),
                                               16, 0, 0);
            }
          }
        }
      };
      const int pre = min(C::NBUF - 1, nchunks);
      for (int c = 0; c < pre; ++c) issue(c);
      loader_wait_barrier(pre - 1);  // chunk 0 landed
      for (int c = 0; c < nchunks; ++c) {
        // chunk c+NBUF-1 reuses the buffer of chunk c-1, consumed before the last barrier
        if (c + C::NBUF - 1 < nchunks) issue(c + C::NBUF - 1);
        const int newest = min(c + C::NBUF - 1, nchunks - 1);
        loader_wait_barrier(newest - (c + 1));  // chunk c+1 landed
      }
      if constexpr (RQ) barrier_lds();  // the compute waves' row-maximum exchange
    }
    return;
  }

  // ---------------- compute waves
  WOperands<NB, GATEUP, NT> wo;
  wo.init(g, shared, ex, tile * CH_WG + wave * CH_WAVE, k_begin, nks, lane);
  wo.rot = krot;

  v8i ring[C::PF][NB];
  v4f acc[MSUB][NB];
  const uint8_t *lds_lane = abuf + lane * 16;
  int pass = 0;
  for (int p0 = 0; p0 < rows; p0 += C::MP, ++pass) {
    const int prow = min(C::MP, rows - p0);
    const int msub = (prow + 15) >> 4;
    const float *rsc = row_scale + (pass & 1) * C::MP;
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[m][nb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < C::PF; ++s) wo.load(ring[s], s);
    barrier_lds();

    for (int ks0 = 0; ks0 < nks_pf; ks0 += C::PF) {
#pragma unroll
      for (int s = 0; s < C::PF; ++s) {
        const int ks = ks0 + s;
        const int c = ks / C::KSC;
        const uint8_t *fa = lds_lane + (c % C::NBUF) * C::BYTES + (ks - c * C::KSC) * 2048;
        // Row groups in batches of MB: a batch's activation fragments are
        // all read from LDS before its MFMAs (groups past msub inside a
        // batch hold the loader's zero pieces).  Two-operand waves only:
        // four-operand ones have no registers to spare.
        constexpr int MB = (NB == 2 && MSUB >= 4) ? 4 : 1;
#pragma unroll
        for (int mb = 0; mb < MSUB; mb += MB) {
          if (mb < msub) {
            v8i a[MB];
#pragma unroll
            for (int j = 0; j < MB; ++j) {
              const v4i a0 = *reinterpret_cast<const v4i *>(fa + (mb + j) * C::KSC * 2048);
              const v4i a1 = *reinterpret_cast<const v4i *>(fa + (mb + j) * C::KSC * 2048 + 1024);
              a[j] = v8i{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            }
            if (MB > 1) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < MB; ++j)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                acc[mb + j][nb] = mfma_e4m3_16x16x128(a[j], ring[s][nb], acc[mb + j][nb]);
          }
        }
        // the pass's last PF steps load nothing (the next pass refills the ring)
        if (ks + C::PF < nks_pf) wo.load(ring[s], ks + C::PF);
        if ((ks + 1) % C::KSC == 0 || ks + 1 == nks_pf) barrier_lds();  // end of chunk c
      }
    }

    // stores stop at the pass's last row that holds a pair
    const int srow = min(max(real - p0, 0), prow);
    if constexpr (RQ) {
      static_assert(GATEUP, "the fused requantisation follows the gate/up GEMM");
      gemm_epilogue_rq<MSUB, NB, NT>(g, acc, wo, rsc, reinterpret_cast<float *>(abuf + C::LDS), row0,
                                     p0, srow, (srow + 15) >> 4, lane, wave, W);
    } else {
      gemm_epilogue<MSUB, NB, GATEUP, NT>(g, acc, wo, rsc, row0, p0, srow, (srow + 15) >> 4, split, lane);
    }
  }
}


// ------------------------------------------------------------------ A-resident grouped GEMM
// Short K (the down projection of small experts, K = f = 192 .. 1408, and the
// gate/up projection of decode batches with few rows per expert): the
// item's activation rows for the WHOLE K range fit in LDS, so the workgroup
// gathers them once and then walks g.ntg consecutive N-tiles of its item.
// Every wave computes (no loader wave), the weight prefetch ring runs on
// across tile boundaries (the next tile's first K steps are in flight during
// the current tile's last steps and epilogue), and after the gather there is
// no workgroup barrier: the A block is read-only.  The weight scales of all
// the workgroup's channels are staged in LDS with the gather, so inside the
// tile loop the only global loads are the weight stream (a load whose result
// is needed early would make the in-order wait drain the prefetched weights).
// The per-tile workgroups of wsgemm_tile pay a gather, a barrier chain and a
// dependent start-up latency for every tile of two to sixteen K steps.
//
// LDS: A fragments [ksp][MSUB] of 2 KB (MFMA operand order, zero for rows
// past the item and K past the end), the rows' activation scales, then the
// channels' weight scales (gate and up interleaved for gate/up).
constexpr int kAresLdsMax = 96 * 1024;
__host__ __device__ constexpr int ares_lds_bytes(int msub, int ksp, int scale_floats) {
  return msub * ksp * 2048 + 16 * msub * 4 + scale_floats * 4;
}

template <int NB, bool GATEUP>
struct TilePtrs {
  const uint8_t *bw[NB];  // tile of K step 0 for channel group nb (wave-uniform)
  int l16;                // lane * 16: the lane's bytes in each 1 KB half
  int ch[NB];
  int nks;
  // c0: the wave's first output channel (no memory access: addresses only)
  __device__ __forceinline__ void set(const GemmArgs &g, bool shared, size_t ex, int c0, int nks_,
                                      int lane) {
    const int N = GATEUP ? g.rs.f : g.rs.d;
    const int K = GATEUP ? g.rs.d : g.rs.f;
    const int KT = (K + 127) >> 7;
    nks = nks_;
    l16 = lane * 16;
    if constexpr (kDebugChecks) dcheck((c0 & 15) == 0, kDbgTile);  // the group clamp below
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int o;
      const uint8_t *wbase;
      if (GATEUP) {
        o = c0 + (nb >> 1) * 16 + (lane & 15);
        wbase = ((nb & 1) == 0 ? (shared ? g.w.ws_gate : g.w.w_gate) : (shared ? g.w.ws_up : g.w.w_up)) +
                ex * (size_t)N * KT * 128;
      } else {
        o = c0 + nb * 16 + (lane & 15);
        wbase = (shared ? g.w.ws_down : g.w.w_down) + ex * (size_t)N * KT * 128;
      }
      ch[nb] = o;
      // c0 and N are multiples of 16: a group past N clamps to the last one
      const int grp = min((c0 >> 4) + (GATEUP ? (nb >> 1) : nb), (N >> 4) - 1);
      bw[nb] = wbase + (size_t)grp * KT * 2048;
    }
  }
  template <bool NT>
  __device__ __forceinline__ void load(v8i (&b)[NB], int ks) const {
    ks = ks < nks ? ks : nks - 1;
    const int o0 = ks * 2048 + l16;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const v4i lo = NT ? load16_nt(bw[nb] + o0) : load16(bw[nb] + o0);
      const v4i hi = NT ? load16_nt(bw[nb] + o0 + 1024) : load16(bw[nb] + o0 + 1024);
      b[nb] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  }
};

template <int MSUB, bool GATEUP, bool NT, int PF>
__device__ __forceinline__ void ares_tile(const GemmArgs &g, int bid, uint8_t *lds) {
  constexpr int NB = 2;
  constexpr int MP = 16 * MSUB;
  constexpr int CH_WAVE = GATEUP ? 8 * NB : 16 * NB;
  const RowSpace &rs = g.rs;
  const int W = __builtin_amdgcn_readfirstlane((int)(blockDim.x >> 6));  // every wave computes
  const int K = GATEUP ? rs.d : rs.f;
  const int N = GATEUP ? rs.f : rs.d;
  const int CH_WG = W * CH_WAVE;
  const int n_tiles = (N + CH_WG - 1) / CH_WG;
  const int n_groups = (n_tiles + g.ntg - 1) / g.ntg;
  const int item_id = bid / n_groups;
  const int t_begin = (bid - item_id * n_groups) * g.ntg;
  const int t_end = min(n_tiles, t_begin + g.ntg);
  int expert, row0, rows, real;
  if (!resolve_item(rs, item_id, expert, row0, rows, real)) return;
  if (t_begin >= t_end) return;
  const int nks = (K + 127) >> 7;
  const int ksp = (nks + PF - 1) / PF * PF;  // K steps padded to the ring depth (zero A)
  const bool shared = expert >= rs.E;
  const size_t ex = (size_t)(shared ? expert - rs.E : expert);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, kg = lane >> 4;
  const int msub = (rows + 15) >> 4;
  float *rsc = reinterpret_cast<float *>(lds + MSUB * ksp * 2048);
  float *wsl = rsc + MP;  // weight scales of channels [t_begin * CH_WG, t_end * CH_WG)
  const int c_first = t_begin * CH_WG;

  // ---- the tiles' first weight steps, then the gather (piece q = (ks, m,
  // half); wave w takes q = w, w + W, ...), the row and weight scales
  TilePtrs<NB, GATEUP> cur, nxt;
  cur.set(g, shared, ex, c_first + wave * CH_WAVE, nks, lane);
  v8i ring[PF][NB];
#pragma unroll
  for (int s = 0; s < PF; ++s) cur.template load<NT>(ring[s], s);
  {
    const uint8_t *arow[MSUB];
#pragma unroll
    for (int m = 0; m < MSUB; ++m) {
      const int r = m * 16 + ln;
      const int grow = row0 + min(r, rows - 1);
      const int sp = rs.sorted_pairs[min(grow, rs.capacity - 1)];
      const int a = act_row<GATEUP>(rs, grow, sp, r < rows);
      arow[m] = a < 0 ? nullptr : g.a + (size_t)a * K;
    }
    const int npieces = ksp * MSUB * 2;
#pragma unroll 4
    for (int q = wave; q < npieces; q += W) {
      const int half = q & 1, m = (q >> 1) % MSUB, ks = (q >> 1) / MSUB;
      const int kb = ks * 128 + half * 64 + kg * 16;
      const uint8_t *base = arow[0];
#pragma unroll
      for (int mm = 1; mm < MSUB; ++mm)
        if (mm == m) base = arow[mm];
      const v4i v = (base && kb < K) ? load16(base + kb) : v4i{0, 0, 0, 0};
      *reinterpret_cast<v4i *>(lds + (ks * MSUB + m) * 2048 + half * 1024 + lane * 16) = v;
    }
    for (int r = threadIdx.x; r < MP; r += blockDim.x) {
      const int grow = row0 + min(r, rows - 1);
      const int sp = rs.sorted_pairs[min(grow, rs.capacity - 1)];
      const int a = act_row<GATEUP>(rs, grow, sp, r < rows);
      rsc[r] = a < 0 ? 0.0f : g.a_scale[a];
    }
    const int nch = (t_end - t_begin) * CH_WG;
    for (int i = threadIdx.x; i < nch; i += blockDim.x) {
      const int o = min(c_first + i, N - 1);
      if (GATEUP) {
        wsl[2 * i] = (shared ? g.w.ss_gate : g.w.s_gate)[ex * N + o];
        wsl[2 * i + 1] = (shared ? g.w.ss_up : g.w.s_up)[ex * N + o];
      } else {
        wsl[i] = (shared ? g.w.ss_down : g.w.s_down)[ex * N + o];
      }
    }
  }
  __syncthreads();

  v4f acc[MSUB][NB];
  const uint8_t *lds_lane = lds + lane * 16;
  for (int t = t_begin; t < t_end; ++t) {
    const bool has_next = t + 1 < t_end;
    if (has_next) nxt.set(g, shared, ex, (t + 1) * CH_WG + wave * CH_WAVE, nks, lane);
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[m][nb] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int ks0 = 0; ks0 < ksp; ks0 += PF) {
#pragma unroll
      for (int s = 0; s < PF; ++s) {
        const int ks = ks0 + s;
        const uint8_t *fa = lds_lane + ks * MSUB * 2048;
        constexpr int MB = MSUB >= 4 ? 4 : MSUB;
#pragma unroll
        for (int mb = 0; mb < MSUB; mb += MB) {
          if (mb < msub) {
            v8i a[MB];
#pragma unroll
            for (int j = 0; j < MB; ++j) {
              const v4i a0 = *reinterpret_cast<const v4i *>(fa + (mb + j) * 2048);
              const v4i a1 = *reinterpret_cast<const v4i *>(fa + (mb + j) * 2048 + 1024);
              a[j] = v8i{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < MB; ++j)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                acc[mb + j][nb] = mfma_e4m3_16x16x128(a[j], ring[s][nb], acc[mb + j][nb]);
          }
        }
        // step ks + PF: this tile's, else the next tile's first steps
        if (ks + PF < ksp)
          cur.template load<NT>(ring[s], ks + PF);
        else if (has_next)
          nxt.template load<NT>(ring[s], ks + PF - ksp);
      }
    }
    // the epilogue's channels and their weight scales (from LDS)
    WOperands<NB, GATEUP, NT> ep;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      ep.ch[nb] = cur.ch[nb];
      const int i = min(cur.ch[nb], N - 1) - c_first;
      ep.wsc[nb] = GATEUP ? wsl[2 * i + (nb & 1)] : wsl[i];
    }
    gemm_epilogue<MSUB, NB, GATEUP, NT>(g, acc, ep, rsc, row0, 0, real, (real + 15) >> 4, 0, lane);
    if (has_next) cur = nxt;
  }
}

// ------------------------------------------------------------------ prefill grouped GEMM
// Row passes of 256 rows (prefill-sized batches re-read an expert's weights
// once per pass, so passes are as tall as registers allow).  Eight waves,
// two per SIMD, and every wave both gathers and computes: wave w gathers row
// groups 2w and 2w+1 of each chunk and computes 16 gate/up channels (32
// down channels) over all 256 rows.  A split into loader and compute waves
// left two SIMDs with one computing wave each.
//
// A chunk is one K step (128 bytes) of the pass's 256 rows, 32 KB of LDS.
// The gather goes through registers: chunk c is loaded at step c-3 into one
// of two staging sets and written to LDS during step c-1, between MFMA
// batches, into the buffer of chunk c-2 (two buffers).  Every load is an
// ordinary one, so the compiler's wait counts stay exact (direct-to-LDS
// loads make it wait for all outstanding loads before the LDS reads).  One
// barrier per step: each wave's LDS writes of chunk t+1 are done, and every
// wave finished chunk t-1, whose buffer the next writes reuse.
struct PfChunk {
  static constexpr int MSUB = 16;
  static constexpr int MP = 16 * MSUB;    // rows per pass
  static constexpr int BYTES = MP * 128;  // one K step of the pass's rows: 32 KB
  static constexpr int PF = 2;            // weight prefetch depth in K steps
  static constexpr int MB = 2;            // row groups per batch of LDS reads (4 measured 6-9 % slower)
  static constexpr int LDS = 2 * BYTES + 2 * MP * (int)sizeof(float);  // + scale table per pass parity
};

template <bool GATEUP, int O16 = -1>
__device__ __forceinline__ void pf_tile(const GemmArgs &g, int bid, uint8_t *abuf) {
  using C = PfChunk;
  constexpr int MSUB = C::MSUB, NB = 2, NW = kPfWaves;
  constexpr int CH_WAVE = GATEUP ? 16 : 32;
  constexpr int CH_WG = NW * CH_WAVE;
  const RowSpace &rs = g.rs;
  const int K = GATEUP ? rs.d : rs.f;
  const int N = GATEUP ? rs.f : rs.d;
  const int n_tiles = (N + CH_WG - 1) / CH_WG;
  const int split = bid % g.splits;
  bid /= g.splits;
  const int tile = bid % n_tiles;
  const int item_id = bid / n_tiles;
  int expert, row0, rows, real;
  if (!resolve_item(rs, item_id, expert, row0, rows, real)) return;
  const int k_begin = split * g.ksplit;
  const int k_end = min(K, k_begin + g.ksplit);
  if (k_begin >= k_end) return;
  const int nks = (k_end - k_begin + 127) >> 7;       // K steps in this split
  const int nch = (nks + C::PF - 1) / C::PF * C::PF;  // chunks (one K step each), a multiple of PF
  const bool shared = expert >= rs.E;
  const size_t ex = (size_t)(shared ? expert - rs.E : expert);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15, kg = lane >> 4;
  float *row_scale = reinterpret_cast<float *>(abuf + 2 * C::BYTES);

  WOperands<NB, GATEUP, false> wo;
  wo.init(g, shared, ex, tile * CH_WG + wave * CH_WAVE, k_begin, nks, lane);

  v8i ring[C::PF][NB];
  v4f acc[MSUB][NB];
  v4i stage[2][4];  // gathered pieces of two chunks: (row group mm, K half p) at 2*mm + p
  int pass = 0;
  for (int p0 = 0; p0 < rows; p0 += C::MP, ++pass) {
    const int prow = min(C::MP, rows - p0);
    const int msub = (prow + 15) >> 4;
    float *rsc = row_scale + (pass & 1) * C::MP;
    // This wave's two row groups (lane ln: row ln of each) and, for waves
    // 0-3, 64 rows of the scale table; lookups issued together.
    const uint8_t *abase[2];
    float tscale = 0.0f;
    {
      int grow[2], sp[2];
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        grow[mm] = row0 + min(p0 + (2 * wave + mm) * 16 + ln, rows - 1);
        sp[mm] = rs.sorted_pairs[min(grow[mm], rs.capacity - 1)];
      }
      const int trow = (wave & 3) * kWave + lane;
      const int tgrow = row0 + min(p0 + trow, rows - 1);
      const int tsp = rs.sorted_pairs[min(tgrow, rs.capacity - 1)];
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int m = 2 * wave + mm;
        const int a = act_row<GATEUP>(rs, grow[mm], sp[mm], m < msub && p0 + m * 16 + ln < rows);
        abase[mm] = a < 0 ? nullptr : g.a + (size_t)a * K;
      }
      const int a = act_row<GATEUP>(rs, tgrow, tsp, trow < prow);
      if (wave < 4 && a >= 0) tscale = g.a_scale[a];
    }
    // Chunk c of this wave's row groups: 16 bytes per lane and piece (row
    // ln, K bytes kg*16 of each 64-byte half); zero past K or for padding.
    auto gather = [&](int c, v4i (&st)[4]) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int kb = k_begin + c * 128 + p * 64 + kg * 16;
          const uint8_t *src = (abase[mm] && kb < k_end) ? abase[mm] + kb : g_zero_piece;
          st[2 * mm + p] = load16(src);
        }
      }
    };
    // ... written where the MFMA reads expect it: fragment m of the chunk
    // at m*2048, its two K halves 1 KB apart, lane l at l*16.
    auto put = [&](int c, const v4i (&st)[4]) {
      uint8_t *dst = abuf + (c & 1) * C::BYTES + lane * 16;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int p = 0; p < 2; ++p)
          *reinterpret_cast<v4i *>(dst + ((2 * wave + mm) * 2 + p) * 1024) = st[2 * mm + p];
    };
#pragma unroll
    for (int m = 0; m < MSUB; ++m)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[m][nb] = v4f{0.f, 0.f, 0.f, 0.f};
    // chunks 0 and 1 (and 2) gathered, chunk 0 written; weights of steps 0, 1
    gather(0, stage[0]);
    gather(1, stage[1]);
    wo.load(ring[0], 0);
    wo.load(ring[1], 1);
    put(0, stage[0]);
    gather(2, stage[0]);
    if (wave < 4) rsc[(wave & 3) * kWave + lane] = tscale;
    barrier_lds();

    for (int ks0 = 0; ks0 < nch; ks0 += C::PF) {
#pragma unroll
      for (int s = 0; s < C::PF; ++s) {
        const int ks = ks0 + s;  // stage[(ks + 1) & 1] holds chunk ks+1
        const uint8_t *fa = abuf + (ks & 1) * C::BYTES + lane * 16;
        // row groups in batches of MB: a batch's fragments are all read from
        // LDS before its MFMAs; chunk ks+1 is written to LDS and chunk ks+3
        // gathered between batches
#pragma unroll
        for (int mb = 0; mb < MSUB; mb += C::MB) {
          if (mb < msub && ks < nks) {  // steps past nks (PF padding) hold zeros
            v8i a[C::MB];
#pragma unroll
            for (int j = 0; j < C::MB; ++j) {
              const v4i a0 = *reinterpret_cast<const v4i *>(fa + (mb + j) * 2048);
              const v4i a1 = *reinterpret_cast<const v4i *>(fa + (mb + j) * 2048 + 1024);
              a[j] = v8i{a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < C::MB; ++j)
#pragma unroll
              for (int nb = 0; nb < NB; ++nb)
                acc[mb + j][nb] = mfma_e4m3_16x16x128(a[j], ring[s][nb], acc[mb + j][nb]);
          }
          __builtin_amdgcn_sched_barrier(0);
          if (mb == 2) put(ks + 1, stage[(ks + 1) & 1]);
          if (mb == 4) gather(ks + 3, stage[(ks + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        wo.load(ring[s], ks + C::PF);
        barrier_lds();
      }
    }
    const int srow = min(max(real - p0, 0), prow);  // stores stop at the last row with a pair
    gemm_epilogue<MSUB, NB, GATEUP, false, O16>(g, acc, wo, rsc, row0, p0, srow, (srow + 15) >> 4, split,
                                                lane);
  }
}


// ------------------------------------------------------------------ down, fp32 products
// No-requant mode: y[row][c] = (sum_o h[row][o] dec(Wd[c][o])) * s_down[c] on
// v_mfma_f32_16x16x4_f32.  Lane l (channel l%16, group kg = l/16) owns, of
// each 128-wide K step, the indices [16kg, +16) and [64 + 16kg, +16) -- the
// two 16-byte pieces of its weight tile -- and instruction q of the step
// takes the q-th of them, for A and B alike.  An accuracy mode: simple
// direct loads, no prefetch pipeline.
// Tile `bid` (= item * ceil(d/64) + channel tile) by 256 threads, tid in
// [0, 256); no workgroup barriers, so a larger workgroup can run several.
__device__ __forceinline__ void down_f32_tile(const GemmArgs &g, int bid, int tid) {
  const RowSpace &rs = g.rs;
  const int d = rs.d, f = rs.f;
  const int KT = (f + 127) >> 7;
  const int n_tiles = (d + 63) >> 6;
  const int item_id = bid / n_tiles;
  const int tile = bid - item_id * n_tiles;
  int expert, row0, rows, real;
  if (!resolve_item(rs, item_id, expert, row0, rows, real)) return;
  const bool shared = expert >= rs.E;
  const size_t ex = (size_t)(shared ? expert - rs.E : expert);
  const uint8_t *wd = (shared ? g.w.ws_down : g.w.w_down) + ex * d * (size_t)KT * 128;
  const float *sd = (shared ? g.w.ss_down : g.w.s_down) + ex * d;
  const int wave = tid >> 6, lane = tid & 63;
  const int ln = lane & 15, kg = lane >> 4;
  const int oc = (tile << 6) + (wave << 4) + ln;
  const uint8_t *bp = wd + (size_t)((oc < d ? oc : d - 1) >> 4) * KT * 2048 + lane * 16;
  const bool half_tail = (f & 127) != 0;
  for (int r0 = 0; r0 < rows; r0 += 16) {
    const int r = r0 + ln;
    const bool aok = r < rows && row_real(rs, row0 + r);
    const float *arow = g.a32 + (size_t)(row0 + (r < rows ? r : 0)) * f + kg * 16;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    for (int ks = 0; ks < KT; ++ks) {
      const bool hi_ok = !(half_tail && ks == KT - 1);  // K past f: zero weights, no A read
      const v4i w0 = load16(bp + ks * 2048);
      const v4i w1 = load16(bp + ks * 2048 + 1024);
      const uint32_t ww[8] = {(uint32_t)w0.x, (uint32_t)w0.y, (uint32_t)w0.z, (uint32_t)w0.w,
                              (uint32_t)w1.x, (uint32_t)w1.y, (uint32_t)w1.z, (uint32_t)w1.w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        v4f av = {0.f, 0.f, 0.f, 0.f};
        if (aok && (q < 4 || hi_ok))
          av = *reinterpret_cast<const v4f *>(arow + ks * 128 + (q < 4 ? 4 * q : 64 + 4 * (q - 4)));
        const v2f lo = e4m3x2_to_f32<false>(ww[q]);
        const v2f hi = e4m3x2_to_f32<true>(ww[q]);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, lo.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, lo.y, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, hi.x, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, hi.y, acc, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = r0 + kg * 4 + i;
      if (rr < rows && oc < d) {
        const int grow = row0 + rr;
        g.out[(size_t)grow * d + oc] = row_real(rs, grow) ? acc[i] * sd[oc] : 0.0f;
      }
    }
  }
}

// ------------------------------------------------------------------ requant
// A workgroup of NT threads requantises one real expert row:
// hq = e4m3(h * 448/amax), sh = amax/448 (the row held in registers).
template <int NT>
__device__ __forceinline__ void requant_row(const RowSpace &rs, const float *__restrict__ h,
                                            uint8_t *__restrict__ hq, float *__restrict__ sh,
                                            int row, float *red) {
  if (!row_real(rs, row)) return;
  constexpr int VEC = (kMaxFfn + NT * 4 - 1) / (NT * 4);
  quantize_row_block<NT, VEC>(h + (size_t)row * rs.f, rs.f, hq + (size_t)row * rs.f, sh + row,
                              red);
}

// One wave requantises one real expert row of up to 64*4*VEC values (the
// row in registers); same arithmetic as requant_row.
template <int VEC>
__device__ __forceinline__ void requant_row_wave(const RowSpace &rs, const float *__restrict__ h,
                                                 uint8_t *__restrict__ hq, float *__restrict__ sh,
                                                 int row, int lane) {
  if (!row_real(rs, row)) return;
  const int f = rs.f;
  const float *x = h + (size_t)row * f;
  v4f v[VEC];
  float amax = 0.0f;
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const int i = (j * kWave + lane) * 4;
    v[j] = i < f ? *reinterpret_cast<const v4f *>(x + i) : v4f{0.f, 0.f, 0.f, 0.f};
    amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
    if constexpr (kDebugChecks) dcheck(finite4(v[j]), kDbgNonFinite);
  }
  amax = wave_max(amax);
  float r = 1.0f, s = 1.0f;
  if (amax != 0.0f) {
    r = kE4m3Max / amax;
    s = amax / kE4m3Max;
  }
  uint8_t *q = hq + (size_t)row * f;
#pragma unroll
  for (int j = 0; j < VEC; ++j) {
    const int i = (j * kWave + lane) * 4;
    if (i < f) *reinterpret_cast<uint32_t *>(q + i) = e4m3x4(v[j].x * r, v[j].y * r, v[j].z * r, v[j].w * r);
  }
  if (lane == 0) sh[row] = s;
}

// ------------------------------------------------------------------ combine
// out[t] = sum_j w[t,j] * y[inv[t,j]] over valid slots in order, then + the
// shared experts' rows in order; each y row is the sum of its K-split slabs
// in split order.  A workgroup of NT threads does NT*4 columns of token t
// starting at column c0.
//
// Slots are taken G at a time: their lookups (ids, inv, w) are requested
// together, then every K-split piece of their rows (up to SM splits), then
// the pieces are added in order -- two memory latencies per group.
// V consecutive y elements as floats: 16-byte loads (4 fp32 or 8 fp16).
template <int V>
struct Cols {
  v4f v[V / 4];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int q = 0; q < V / 4; ++q) v[q] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ void add(const Cols &o) {
#pragma unroll
    for (int q = 0; q < V / 4; ++q) v[q] += o.v[q];
  }
  __device__ __forceinline__ void fma(float w, const Cols &o) {
#pragma unroll
    for (int q = 0; q < V / 4; ++q) v[q] += w * o.v[q];
  }
};
template <typename Y>
constexpr int cols_per_load() { return 4; }

__device__ __forceinline__ Cols<4> load_cols(const float *p) {
  Cols<4> c;
  c.v[0] = *reinterpret_cast<const v4f *>(p);
  return c;
}
__device__ __forceinline__ Cols<4> load_cols(const _Float16 *p) {
  typedef _Float16 v4h __attribute__((ext_vector_type(4)));
  const v4h h = *reinterpret_cast<const v4h *>(p);
  Cols<4> c;
  c.v[0] = v4f{(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
  return c;
}

template <int G, int SM, typename Y>
__device__ __forceinline__ Cols<cols_per_load<Y>()> combine_groups(
    const RowSpace &rs, const Y *__restrict__ y, int splits, const int32_t *__restrict__ ids,
    const float *__restrict__ w, const int32_t *__restrict__ inv, int t, int c) {
  constexpr int V = cols_per_load<Y>();
  const int d = rs.d, K = rs.k_max, J = K + rs.S;  // routed slots, then the shared rows
  const size_t slab = (size_t)(rs.capacity + rs.S * rs.T) * d;
  Cols<V> acc;
  acc.zero();
  for (int j0 = 0; j0 < J; j0 += G) {
    int row[G];
    float wt[G];
    bool ok[G];
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int j = j0 + u;
      if (j < K) {
        const int p = t * K + j;
        const int id = ids[p], r = inv[p];
        wt[u] = w[p];
        ok[u] = id >= 0;
        // a slot's row lies in [0, capacity) (checked in the debug build)
        if constexpr (kDebugChecks) ok[u] = ok[u] && dcheck(r >= 0 && r < rs.capacity, kDbgRow);
        row[u] = ok[u] ? r : 0;
      } else {  // a shared row (weight 1: 1 * x == x), or past the end
        wt[u] = 1.0f;
        ok[u] = j < J;
        row[u] = j < J ? rs.capacity + (j - K) * rs.T + t : 0;
      }
    }
    Cols<V> v[G][SM];
#pragma unroll
    for (int u = 0; u < G; ++u)
#pragma unroll
      for (int sp = 0; sp < SM; ++sp)  // uniform conditions
        if (j0 + u < J && sp < splits) v[u][sp] = load_cols(y + sp * slab + (size_t)row[u] * d + c);
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (j0 + u < J) {
        Cols<V> cur = v[u][0];
#pragma unroll
        for (int sp = 1; sp < SM; ++sp)
          if (sp < splits) cur.add(v[u][sp]);
        if (ok[u]) acc.fma(wt[u], cur);
      }
    }
  }
  return acc;
}

// fp16 y in one slab (splits == 1): columns [c0, c0 + NT * 8) of token t, 16
// bytes of each row per thread.  A slot's validity is the same for the whole
// workgroup (no divergence); rows are added in slot order, then the shared
// experts' -- the operations and their order are those of combine_groups, so
// both give the same sums bit for bit.
template <int NT, int SL>
__device__ __forceinline__ void combine_row16(const RowSpace &rs, const _Float16 *__restrict__ y,
                                              const int32_t *__restrict__ ids,
                                              const float *__restrict__ w,
                                              const int32_t *__restrict__ inv,
                                              float *__restrict__ out, int t, int c0) {
  const int d = rs.d, K = rs.k_max;
  const int lane = (int)threadIdx.x & 63;
  // Every slot's lookups at once: lane j of each wave holds slot j's row and
  // weight (k_max <= 32), the valid slots are a ballot; then their rows are
  // requested SL at a time (wave-uniform row indices from v_readlane) and
  // added in slot order, then the shared experts' rows -- the same sums as
  // slot-by-slot, in one lookup latency plus one per SL valid slots.
  int my_row = 0;
  float my_w = 0.0f;
  bool my_ok = false;
  if (lane < K) {
    const int p = t * K + lane;
    const int id = ids[p], r = inv[p];
    my_w = w[p];
    my_ok = id >= 0;
    if constexpr (kDebugChecks) my_ok = my_ok && dcheck(r >= 0 && r < rs.capacity, kDbgRow);
    my_row = my_ok ? r : 0;
  }
  uint64_t pending = __builtin_amdgcn_ballot_w64(my_ok);
  const int c = c0 + (int)threadIdx.x * 8;
  const bool live = c < d;
  Cols<8> acc;
  acc.zero();
  auto add_rows = [&](const int (&row)[SL], const float (&wt)[SL], int n) {
    v8h v[SL];
#pragma unroll
    for (int u = 0; u < SL; ++u)
      if (u < n && live) v[u] = *reinterpret_cast<const v8h *>(y + (size_t)row[u] * d + c);
#pragma unroll
    for (int u = 0; u < SL; ++u) {
      if (u < n) {
        Cols<8> cur;
#pragma unroll
        for (int q = 0; q < 2; ++q)
          cur.v[q] = v4f{(float)v[u][4 * q], (float)v[u][4 * q + 1], (float)v[u][4 * q + 2],
                         (float)v[u][4 * q + 3]};
        acc.fma(wt[u], cur);
      }
    }
  };
  while (pending) {  // routed slots, ascending
    int row[SL];
    float wt[SL];
    int n = 0;
#pragma unroll
    for (int u = 0; u < SL; ++u) {
      row[u] = 0;
      wt[u] = 0.0f;
      if (pending) {
        const int j = (int)__builtin_ctzll(pending);
        pending &= pending - 1;
        row[u] = readlane(my_row, j);
        wt[u] = readlane(my_w, j);
        n = u + 1;
      }
    }
    add_rows(row, wt, n);
  }
  for (int s0 = 0; s0 < rs.S; s0 += SL) {  // shared experts, weight 1 (1 * x == x)
    int row[SL];
    float wt[SL];
    const int n = min(SL, rs.S - s0);
#pragma unroll
    for (int u = 0; u < SL; ++u) {
      row[u] = rs.capacity + (s0 + u) * rs.T + t;
      wt[u] = 1.0f;
    }
    add_rows(row, wt, n);
  }
  if (!live) return;
#pragma unroll
  for (int q = 0; q < 2; ++q)
    *reinterpret_cast<v4f *>(out + (size_t)t * rs.d + c + 4 * q) = acc.v[q];
}

// Columns [c0, c0 + NT * cols_per_load<Y>()) of token t.
template <int NT, typename Y>
__device__ __forceinline__ void combine_chunk(const RowSpace &rs, const Y *__restrict__ y,
                                              int splits, const int32_t *__restrict__ ids,
                                              const float *__restrict__ w,
                                              const int32_t *__restrict__ inv,
                                              float *__restrict__ out, int t, int c0) {
  constexpr int V = cols_per_load<Y>();
  const int c = c0 + threadIdx.x * V;
  if (c >= rs.d) return;
  // registers for the loads of a slot group: G slots x SM split pieces
  const Cols<V> acc = splits == 1  ? combine_groups<8, 1>(rs, y, splits, ids, w, inv, t, c)
                      : splits <= 2 ? combine_groups<8, 2>(rs, y, splits, ids, w, inv, t, c)
                                    : combine_groups<2, kMaxDownSplits>(rs, y, splits, ids, w, inv, t, c);
#pragma unroll
  for (int q = 0; q < V / 4; ++q)
    *reinterpret_cast<v4f *>(out + (size_t)t * rs.d + c + 4 * q) = acc.v[q];
}

}  // namespace fp8moe
