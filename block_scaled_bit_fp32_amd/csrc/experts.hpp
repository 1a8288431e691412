// Dequant-fused expert GEMVs for gfx950: gate/up with SwiGLU, down.
//
//   gateup_kernel  every lane holds a gate row and the matching up row, so SwiGLU is
//                  applied in registers; h goes to the workspace.
//   down_kernel    partial outputs o (per pair and hidden row) go to the workspace.
// Work is cut into units: one expert (or the shared expert) with a group of at most NG
// of its tokens, i.e. a sequence of row-steps over the expert's rows. Both kernels are
// persistent: a few resident workgroups per CU each take a contiguous range of equal
// cost over all units (shared expert first, then the selected experts in id order).
// One wave builds the per-expert tables from topk_ids with ballots and one scan; every
// workgroup then finds its first unit in closed form and issues its first weight loads
// before it stages the activations (and scales) of as many of its units as fit in LDS.
// Weight rows then stream with the 16-byte pieces of the next step (possibly of the
// next unit) in flight while the current step computes; the last step prefetches
// nothing. Weights are decoded in registers with the gfx950 FP4/FP8
// converts. Workgroups never exchange data inside a launch: the h re-quantization and
// the combine are separate launches (combine.hip).
#pragma once
#include <algorithm>
#include <type_traits>

#include "launch.hpp"
#include "rows.hpp"
#include "span.hpp"
#include "topk.hpp"

namespace moe {

// ====================================================================== LDS layout
// Per-expert tables of one class (routed experts, or the shared expert alone). Units of
// an expert are its groups of at most NG tokens, in token order; class rows list the
// tokens of every expert, experts in increasing id order.
struct ClassTab {
  int* ex_id;    // [A] expert id (0 for the shared expert)
  int* ex_n;     // [A] tokens of the expert
  int* ex_row;   // [A + 1] exclusive prefix of tokens: the expert's first class row
  int* ex_unit;  // [A + 1] exclusive prefix of units
  int* ex_cost;  // [A + 1] exclusive prefix of cost (steps * (cw * units + ct * tokens))
  int* r_tok;    // [rows] token of each class row
  int* r_pair;   // [rows] its pair index (t*k + j; the shared expert uses T*k + t)
  int* r_exp;    // [rows] its expert
  int A;         // experts in the class
};

struct ExpertLds {
  uint64_t* tmask;  // [E][NW] token mask of each expert, NW = ceil(T / 64) words
  int nw;
  int* first;       // [E] first pair (t*k + j) naming each expert
  int* ebase;       // [E] first routed class row of each selected expert
  int* ids;         // [T*k] topk_ids
  int* nA;          // [4] selected expert count
  int* span;        // [8] this workgroup's Span (routed workgroups)
  ClassTab rt, sh;
  float* w_gs;      // [2 * kWinRows] global weight scales of the staged rows' experts
  float* w_tsc;     // [kWinRows] activation scales of the staged rows
  float* gs_rt;     // [2 * E] global weight scales of the routed experts (narrow token items)
  float* gs_sh;     // [2] those of the shared expert (token items)
  uint8_t* tile;    // activations of the staged rows, K * esize bytes each
};

__device__ __forceinline__ ExpertLds carve(const ExpertArgs& a, uint8_t* smem) {
  ExpertLds L;
  const int P = a.T * a.k, Am = routed_capacity(a.E, P);
  L.nw = (a.T + 63) / 64;
  L.tmask = reinterpret_cast<uint64_t*>(smem);
  L.first = reinterpret_cast<int*>(L.tmask + a.E * L.nw);
  L.ebase = L.first + a.E;
  L.ids = L.ebase + a.E;
  L.nA = L.ids + P;
  L.span = L.nA + 4;
  int* q = L.span + 8;
  auto tab = [&](ClassTab& C, int A, int rows) {
    C.ex_id = q; q += A;
    C.ex_n = q; q += A;
    C.ex_row = q; q += A + 1;
    C.ex_unit = q; q += A + 1;
    C.ex_cost = q; q += A + 1;
    C.r_tok = q; q += rows;
    C.r_pair = q; q += rows;
    C.r_exp = q; q += rows;
    C.A = 0;
  };
  tab(L.rt, Am, P);
  tab(L.sh, 1, a.T);
  L.w_gs = reinterpret_cast<float*>(q);
  L.w_tsc = L.w_gs + 2 * kWinRows;
  L.gs_rt = L.w_tsc + kWinRows;
  L.gs_sh = L.gs_rt + 2 * a.E;
  L.tile = smem + a.lds_list_bytes;
  return L;
}

// ===================================================================== GEMV core
template <int FMT>
__device__ __forceinline__ int64_t elem_byte(int el) {
  return FMT == W_BF16 ? 2 * (int64_t)el : (FMT == W_MXFP8 ? (int64_t)el : (int64_t)(el >> 1));
}

// LDS byte offset of 16-byte sub-piece `sub` of piece `pc` (pc = s * LPR + jl): the
// sub-pieces of all lanes of a row are consecutive, so a wave's reads are conflict-free
// and the G rows of a wave read the same addresses (broadcast).
__device__ __forceinline__ int act_slot(int pc, int sub, int nsub, int LPR) {
  const int jl = pc % LPR, pass = pc / LPR;
  return ((pass * nsub + sub) * LPR + jl) * 16;
}

// Staging of nt activation rows (all K elements each) into the LDS tile.
//   AK = 0: BF16 values (exact), 8 per 16-byte slot;  AK = 1: FP32 values, 4 per slot.
// Slot u of the rows is row u / units, element (u % units) * PER. The quotient is
// taken in FP32 from (u + 1/2) / units, exact here: u < 2^16 and the fraction is at
// least 1/(2 units) away from an integer.
template <int AK>
struct SlotMap {
  static constexpr int PER = AK == 0 ? 8 : 4;
  int units, lg, tstride;
  float inv;
  __device__ __forceinline__ SlotMap(const GemvMap& m, int K)
      : units(K / PER), lg(__builtin_ctz(m.LPR)), tstride(K * m.esize), inv(1.0f / (float)(K / PER)) {}
  __device__ __forceinline__ int row(int u) const { return (int)(((float)u + 0.5f) * inv); }
  __device__ __forceinline__ int elem(int u, int t) const { return (u - t * units) * PER; }
  // LDS byte offset (see act_slot) of slot u in row t
  template <int EPL>
  __device__ __forceinline__ int offset(int t, int el) const {
    constexpr int NSUB = EPL / PER;
    const int pc = el / EPL, sub = (el % EPL) / PER;
    return t * tstride + ((((pc >> lg) * NSUB + sub) << lg) + (pc & ((1 << lg) - 1))) * 16;
  }
};

template <int AK, int EPL, class Ld, class Cv>
__device__ __forceinline__ void stage_tile(uint8_t* tile, const GemvMap& m, int K, int nt, Ld ld, Cv cv) {
  const SlotMap<AK> sm(m, K);
  for (int u = threadIdx.x; u < nt * sm.units; u += kBlock) {
    const int t = sm.row(u), el = sm.elem(u, t);
    *reinterpret_cast<uint4*>(tile + sm.template offset<EPL>(t, el)) = cv(ld(t, el));
  }
}

// The same in two phases with the raw slots parked in registers (at most kPreSlots per
// thread): the loads are issued before the first weight loads and stored afterwards, so
// waiting for them never waits for weight bytes (vector-memory counters retire in order).
// Slots per thread: 4 for gate/up (a 4 KB token row takes one), 12 for down windows,
// kTokParkBytes / 4 KB for the token walk.
constexpr int kPreSlots = 12;
constexpr int kPreSlotsGateup = 4;
constexpr int kPreSlotsTok = kTokParkBytes / (kBlock * 16);
// Every slot issues its load (slots past the rows re-read the last one): one basic block,
// no per-slot branches. An empty first window (a row longer than the slots: nt = 0)
// parks nothing; the walk stages it instead.
template <int AK, int NS, class Ld>
__device__ __forceinline__ void park_rows(const SlotMap<AK>& sm, int nt, Ld ld, uint4 (&raw)[NS]) {
  if (nt <= 0) return;
  const int n = nt * sm.units;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int u = min(i * kBlock + (int)threadIdx.x, n - 1);
    const int t = sm.row(u);
    raw[i] = ld(t, sm.elem(u, t));
  }
}
template <int AK, int EPL, int NS, class Cv>
__device__ __forceinline__ void unpark_rows(const SlotMap<AK>& sm, uint8_t* tile, int nt, Cv cv,
                                            const uint4 (&raw)[NS]) {
  if (nt <= 0) return;
  const int n = nt * sm.units;
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int u = i * kBlock + threadIdx.x;
    if (u < n) {
      const int t = sm.row(u);
      *reinterpret_cast<uint4*>(tile + sm.template offset<EPL>(t, sm.elem(u, t))) = cv(raw[i]);
    }
  }
}

// acc[q][t] += row_q(piece) . act(t, piece) for one 16-byte weight piece per row.
template <int FMT, int AK, int NT, int RPL>
__device__ __forceinline__ void accumulate_piece(const uint4 (&wv)[RPL], const uint32_t (&sv)[RPL],
                                                 const uint8_t* tile, int tstride, int LPR, int s,
                                                 int jl, float (&acc)[RPL][4]) {
  constexpr int EPL = elems_per_piece(FMT);
  constexpr int NSUB = AK == 0 ? EPL / 8 : EPL / 4;
  const uint8_t* base = tile + ((s * NSUB) * LPR + jl) * 16;
  const int sstride = LPR * 16;  // next sub-piece of the same piece
  // BF16 activations: every token's sub-pieces of this piece are read once, up front, for
  // all RPL rows (into registers of their own, so the LDS reads overlap)
  constexpr int NSA = AK == 0 ? NSUB : 1;
  uint4 ab[NT][NSA];
  if constexpr (AK == 0) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int sb = 0; sb < NSA; ++sb) ab[t][sb] = *reinterpret_cast<const uint4*>(base + t * tstride + sb * sstride);
  }
#pragma unroll
  for (int q = 0; q < RPL; ++q) {
    const uint32_t w[4] = {wv[q].x, wv[q].y, wv[q].z, wv[q].w};
    if constexpr (AK == 0) {
      if constexpr (FMT == W_NVFP4 || FMT == W_MXFP4) {
        const float sc = FMT == W_MXFP4 ? e8m0_to_f32(sv[q] & 0xFFu) : 1.0f;
        uint32_t wb[16];
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          wb[4 * wi + 0] = as_u32(fp4x2_to_bf16<0>(w[wi], sc));
          wb[4 * wi + 1] = as_u32(fp4x2_to_bf16<1>(w[wi], sc));
          wb[4 * wi + 2] = as_u32(fp4x2_to_bf16<2>(w[wi], sc));
          wb[4 * wi + 3] = as_u32(fp4x2_to_bf16<3>(w[wi], sc));
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint4 a0 = ab[t][0], a1 = ab[t][1], a2 = ab[t][2], a3 = ab[t][3];
          float p0 = 0.0f, p1 = 0.0f;
          p0 = dot2(wb[0], a0.x, p0); p0 = dot2(wb[1], a0.y, p0);
          p0 = dot2(wb[2], a0.z, p0); p0 = dot2(wb[3], a0.w, p0);
          p0 = dot2(wb[4], a1.x, p0); p0 = dot2(wb[5], a1.y, p0);
          p0 = dot2(wb[6], a1.z, p0); p0 = dot2(wb[7], a1.w, p0);
          p1 = dot2(wb[8], a2.x, p1); p1 = dot2(wb[9], a2.y, p1);
          p1 = dot2(wb[10], a2.z, p1); p1 = dot2(wb[11], a2.w, p1);
          p1 = dot2(wb[12], a3.x, p1); p1 = dot2(wb[13], a3.y, p1);
          p1 = dot2(wb[14], a3.z, p1); p1 = dot2(wb[15], a3.w, p1);
          if constexpr (FMT == W_NVFP4) {
            acc[q][t] = fmaf(p0, e4m3_to_f32(sv[q] & 0xFFu), acc[q][t]);
            acc[q][t] = fmaf(p1, e4m3_to_f32((sv[q] >> 8) & 0xFFu), acc[q][t]);
          } else {
            acc[q][t] += p0 + p1;
          }
        }
      } else if constexpr (FMT == W_MXFP8) {
        const float sc = e8m0_to_f32(sv[q] & 0xFFu);
        uint32_t wb[8];
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          wb[2 * wi] = as_u32(fp8x2_to_bf16<false>(w[wi], sc));
          wb[2 * wi + 1] = as_u32(fp8x2_to_bf16<true>(w[wi], sc));
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint4 a0 = ab[t][0], a1 = ab[t][1];
          float r = acc[q][t];
          r = dot2(wb[0], a0.x, r); r = dot2(wb[1], a0.y, r);
          r = dot2(wb[2], a0.z, r); r = dot2(wb[3], a0.w, r);
          r = dot2(wb[4], a1.x, r); r = dot2(wb[5], a1.y, r);
          r = dot2(wb[6], a1.z, r); r = dot2(wb[7], a1.w, r);
          acc[q][t] = r;
        }
      } else {  // BF16 weights
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint4 a0 = ab[t][0];
          float r = acc[q][t];
          r = dot2(w[0], a0.x, r); r = dot2(w[1], a0.y, r);
          r = dot2(w[2], a0.z, r); r = dot2(w[3], a0.w, r);
          acc[q][t] = r;
        }
      }
    } else {  // FP32 activations (all of a piece's LDS reads are issued before the first
              // use, into registers of their own, so that they overlap)
      if constexpr (FMT == W_NVFP4 || FMT == W_MXFP4) {
        const float sc = FMT == W_MXFP4 ? e8m0_to_f32(sv[q] & 0xFFu) : 1.0f;
        float4 av[NT][8];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int sb = 0; sb < 8; ++sb) av[t][sb] = *reinterpret_cast<const float4*>(base + t * tstride + sb * sstride);
#pragma unroll
        for (int half = 0; half < 2; ++half) {  // elements 16*half .. 16*half + 15
          float wf[16];
#pragma unroll
          for (int wj = 0; wj < 2; ++wj) {
            const uint32_t ww = w[2 * half + wj];
            const f32x2_t v0 = fp4x2_to_f32<0>(ww, sc), v1 = fp4x2_to_f32<1>(ww, sc);
            const f32x2_t v2 = fp4x2_to_f32<2>(ww, sc), v3 = fp4x2_to_f32<3>(ww, sc);
            wf[8 * wj + 0] = v0.x; wf[8 * wj + 1] = v0.y; wf[8 * wj + 2] = v1.x; wf[8 * wj + 3] = v1.y;
            wf[8 * wj + 4] = v2.x; wf[8 * wj + 5] = v2.y; wf[8 * wj + 6] = v3.x; wf[8 * wj + 7] = v3.y;
          }
          const float S = FMT == W_NVFP4 ? e4m3_to_f32((sv[q] >> (8 * half)) & 0xFFu) : 1.0f;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            float pp = 0.0f;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
              const float4 v = av[t][4 * half + sb];
              pp = fmaf(wf[4 * sb + 0], v.x, pp);
              pp = fmaf(wf[4 * sb + 1], v.y, pp);
              pp = fmaf(wf[4 * sb + 2], v.z, pp);
              pp = fmaf(wf[4 * sb + 3], v.w, pp);
            }
            acc[q][t] = FMT == W_NVFP4 ? fmaf(pp, S, acc[q][t]) : acc[q][t] + pp;
          }
        }
      } else if constexpr (FMT == W_MXFP8) {
        const float sc = e8m0_to_f32(sv[q] & 0xFFu);
        float wf[16];
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          f32x2_t lo = fp8x2_to_f32<false>(w[wi], sc), hi = fp8x2_to_f32<true>(w[wi], sc);
          wf[4 * wi + 0] = lo.x; wf[4 * wi + 1] = lo.y; wf[4 * wi + 2] = hi.x; wf[4 * wi + 3] = hi.y;
        }
        float4 av[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int sb = 0; sb < 4; ++sb) av[t][sb] = *reinterpret_cast<const float4*>(base + t * tstride + sb * sstride);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float r = acc[q][t];
#pragma unroll
          for (int sb = 0; sb < 4; ++sb) {
            const float4 v = av[t][sb];
            r = fmaf(wf[4 * sb + 0], v.x, r); r = fmaf(wf[4 * sb + 1], v.y, r);
            r = fmaf(wf[4 * sb + 2], v.z, r); r = fmaf(wf[4 * sb + 3], v.w, r);
          }
          acc[q][t] = r;
        }
      } else {  // BF16 weights
        float wf[8];
#pragma unroll
        for (int wi = 0; wi < 4; ++wi) {
          wf[2 * wi] = __uint_as_float(w[wi] << 16);
          wf[2 * wi + 1] = __uint_as_float(w[wi] & 0xFFFF0000u);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint8_t* p = base + t * tstride;
          const float4 a0 = *reinterpret_cast<const float4*>(p);
          const float4 a1 = *reinterpret_cast<const float4*>(p + sstride);
          float r = acc[q][t];
          r = fmaf(wf[0], a0.x, r); r = fmaf(wf[1], a0.y, r); r = fmaf(wf[2], a0.z, r); r = fmaf(wf[3], a0.w, r);
          r = fmaf(wf[4], a1.x, r); r = fmaf(wf[5], a1.y, r); r = fmaf(wf[6], a1.z, r); r = fmaf(wf[7], a1.w, r);
          acc[q][t] = r;
        }
      }
    }
  }
}

// Raw weight pieces of one pipeline step for this lane: NPB pieces x RPL rows.
template <int RPL>
struct WeightRegs {
  static constexpr int NPB = 4;
  uint4 w[NPB][RPL];
  uint32_t s[NPB][RPL];
  uint4 sc;   // NVFP4: 16 bytes of the batch's scales of the wave's rows (ScaleChunk)
};

// NVFP4 block scales of a batch (E4M3, one per 16 elements), one 16-byte load per lane
// instead of one 2-byte load per piece and row (MX scales, one byte per piece, stay
// per-piece loads). The batch's pieces of a row are one contiguous run of its scale row,
// bb = NPB x LPR x 2 bytes at b x bb; the wave's G rows of one q hold G x bb = 128 x NPB
// bytes, RPL x that is at most 1 KB. Lane c loads chunk c of them (clamped to the last)
// and writes it to the wave's own 1 KB of LDS, where each lane then reads its pieces'
// scales (a wave's LDS operations complete in order: no barrier). With one batch per row
// the G rows are contiguous and a chunk may span rows; with several, bb is a multiple of
// 16 (the host checks) and a chunk lies in one row. ScaleChunk is the lane's constant
// part of the address: which q, the wave's first row relative to the lane's own, the
// offset from that row's start.
struct ScaleChunk {
  int q, drow, off;
  int bb;       // bytes of a row's scales per batch
  int qbytes;   // bytes of one q's staged rows (G x bb)
};
template <int FMT, int RPL>
__device__ __forceinline__ ScaleChunk scale_chunk(const GemvMap& m, int64_t scale_row_bytes) {
  constexpr int EPL = elems_per_piece(FMT);
  const int lane = threadIdx.x & (kWave - 1);
  const int bb = (m.NPB * m.LPR * EPL) >> 4;
  const int qbytes = m.G * bb, cpq = qbytes >> 4;
  const int c = min(lane, RPL * cpq - 1);
  const int q = RPL == 2 && c >= cpq ? 1 : 0;
  const int cc = c - q * cpq;
  int off = cc * 16;
  if (m.NB > 1) {
    const int cpr = bb >> 4, crow = cc / cpr;
    off = crow * (int)scale_row_bytes + (cc - crow * cpr) * 16;
  }
  return ScaleChunk{q, -(lane >> m.lg), off, bb, qbytes};
}

// Loads batch b (pieces b*NPB .. b*NPB + NPB - 1) of the lane's rows. Always issues
// exactly NPB_max x RPL weight loads (slots beyond the batch reload its first piece) and,
// for NVFP4, one scale chunk: a step-independent count lets the compiler
// wait for one step's loads while the next step's are still in flight (vector-memory
// counters retire in issue order).
template <int FMT, int RPL>
__device__ __forceinline__ void fetch_batch(const WTensor& W, const GemvMap& m, const int64_t (&rows)[RPL],
                                            int b, int jl, const ScaleChunk& sk, WeightRegs<RPL>& R) {
  constexpr int EPL = elems_per_piece(FMT);
#pragma unroll
  for (int q = 0; q < RPL; ++q) {
    const uint8_t* rp = W.codes + rows[q] * W.code_row_bytes;
    const uint8_t* sp = W.scales ? W.scales + rows[q] * W.scale_row_bytes : nullptr;
#pragma unroll
    for (int i = 0; i < WeightRegs<RPL>::NPB; ++i) {
      const int ii = i < m.NPB ? i : 0;
      const int el = ((b * m.NPB + ii) * m.LPR + jl) * EPL;
      R.w[i][q] = load_stream16(rp + elem_byte<FMT>(el));
      if constexpr (FMT == W_MXFP4 || FMT == W_MXFP8)
        R.s[i][q] = sp[el >> 5];
      else
        R.s[i][q] = 0u;   // (NVFP4: from the staged chunk)
    }
  }
  if constexpr (FMT == W_NVFP4) {
    const int64_t r = (sk.q ? rows[RPL - 1] : rows[0]) + sk.drow;
    R.sc = load_stream16(W.scales + r * W.scale_row_bytes + sk.off + b * sk.bb);
  }
}

// ===================================================================== work walk
// A walk position: batch b of row-step s of group g of the class's expert index a
// (expert id e with n tokens, first class row rb).
struct Cursor {
  int a, g, s, b;
  int e, n, rb;
};

// The shared expert's class: one expert with all T tokens (no synchronization; the
// routed build that follows synchronizes).
__device__ __forceinline__ void build_shared(const ExpertArgs& a, ClassTab& C, int NG, int steps, int cw,
                                             int ct) {
  const int units = (a.T + NG - 1) / NG;
  if (threadIdx.x == 0) {
    C.ex_id[0] = 0;
    C.ex_n[0] = a.T;
    C.ex_row[0] = 0; C.ex_row[1] = a.T;
    C.ex_unit[0] = 0; C.ex_unit[1] = units;
    C.ex_cost[0] = 0; C.ex_cost[1] = steps * (cw * units + ct * a.T);
  }
  for (int t = threadIdx.x; t < a.T; t += kBlock) {
    C.r_tok[t] = t;
    C.r_pair[t] = a.T * a.k + t;
    C.r_exp[t] = 0;
  }
  C.A = 1;
}

// Tokens of expert e, and the rank of token t among them (token masks in LDS).
__device__ __forceinline__ int tok_count(const ExpertLds& L, int e) {
  int n = 0;
  for (int w = 0; w < L.nw; ++w) n += __popcll(L.tmask[e * L.nw + w]);
  return n;
}
__device__ __forceinline__ int tok_rank(const ExpertLds& L, int e, int t) {
  int r = __popcll(L.tmask[e * L.nw + (t >> 6)] & ((1ull << (t & 63)) - 1ull));
  for (int w = 0; w < (t >> 6); ++w) r += __popcll(L.tmask[e * L.nw + w]);
  return r;
}

// The routed class from topk_ids (synchronizes). The selected experts are taken in the
// order of their first pair (t*k + j): an expert's first pair is its leader, so wave 0
// scans the T*k pairs, 64 at a time, rather than all E experts: a first pass sums the
// tokens, units and costs of the leaders, a second takes the prefix sums (DPP scans),
// writes the compacted tables and locates the span of routed workgroup b of G, which
// it leaves in L.span. Entries outside [0, E) are ignored. Class rows are filled by
// build_rows.
__device__ __forceinline__ void build_routed(const ExpertArgs& a, const ExpertLds& L, ClassTab& C,
                                             const ClassCost& k, int NB, int b, int G) {
  const int P = a.T * a.k;
  for (int i = threadIdx.x; i < a.E * L.nw; i += kBlock) L.tmask[i] = 0ull;
  for (int i = threadIdx.x; i < a.E; i += kBlock) L.first[i] = 0x7FFFFFFF;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += kBlock) {
    const int e = a.ids[p];
    L.ids[p] = e;
    if ((unsigned)e < (unsigned)a.E) {
      const int t = p / a.k;
      atomicOr(reinterpret_cast<unsigned long long*>(&L.tmask[e * L.nw + (t >> 6)]), 1ull << (t & 63));
      atomicMin(&L.first[e], p);
    }
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const uint64_t below = (1ull << lane) - 1ull;
    // one pair per lane: its expert, whether it leads it, and the leader's counts
    auto pair_at = [&](int c0, int& e, bool& ld, int& nu, int& cost) {
      const int p = c0 + lane;
      e = p < P ? L.ids[p] : -1;
      ld = (unsigned)e < (unsigned)a.E && L.first[e] == p;
      const int n = ld ? tok_count(L, e) : 0;
      const int u = (n + k.NG - 1) / k.NG;
      nu = n | (u << 16);
      cost = k.steps * (k.cw * u + k.ct * n);
    };
    int tnu = 0, tc = 0, A = 0;
    for (int c0 = 0; c0 < P; c0 += kWave) {
      int e, nu, cost;
      bool ld;
      pair_at(c0, e, ld, nu, cost);
      tnu += __builtin_amdgcn_readlane(wave_incl_sum(nu), kWave - 1);
      tc += __builtin_amdgcn_readlane(wave_incl_sum(cost), kWave - 1);
      A += __popcll(__ballot(ld));
    }
    int c_lo, c_hi;
    wg_share(tc, b, G, ShareW{a.sh_wgs, a.ncu, a.late16}, c_lo, c_hi);
    const Located end{A, 0, tc, tnu >> 16, tnu & 0xFFFF, -1};
    Located lo = end, hi = end;
    int bnu = 0, bc = 0, ba = 0;
    for (int c0 = 0; c0 < P; c0 += kWave) {
      int e, cnu, ccost;
      bool ld;
      pair_at(c0, e, ld, cnu, ccost);
      const uint64_t lead = __ballot(ld);
      const int inu = wave_incl_sum(cnu), ic = wave_incl_sum(ccost);
      const int xnu = bnu + inu - cnu, xc = bc + ic - ccost;   // exclusive
      const int n = cnu & 0xFFFF;
      const int i = ba + __popcll(lead & below);
      if (ld) {
        C.ex_id[i] = e;
        C.ex_n[i] = n;
        C.ex_row[i] = xnu & 0xFFFF;
        C.ex_unit[i] = xnu >> 16;
        C.ex_cost[i] = xc;
        L.ebase[e] = xnu & 0xFFFF;
      }
      const uint64_t blo = __ballot(ld && xc <= c_lo), bhi = __ballot(ld && xc <= c_hi);
      if (blo && c_lo < tc) {
        const int j = 63 - __clzll(blo);
        lo = Located{__builtin_amdgcn_readlane(i, j), __builtin_amdgcn_readlane(n, j),
                     __builtin_amdgcn_readlane(xc, j), __builtin_amdgcn_readlane(xnu >> 16, j),
                     __builtin_amdgcn_readlane(xnu & 0xFFFF, j), __builtin_amdgcn_readlane(e, j)};
      }
      if (bhi && c_hi < tc) {
        const int j = 63 - __clzll(bhi);
        hi = Located{__builtin_amdgcn_readlane(i, j), __builtin_amdgcn_readlane(n, j),
                     __builtin_amdgcn_readlane(xc, j), __builtin_amdgcn_readlane(xnu >> 16, j),
                     __builtin_amdgcn_readlane(xnu & 0xFFFF, j), __builtin_amdgcn_readlane(e, j)};
      }
      bnu += __builtin_amdgcn_readlane(inu, kWave - 1);
      bc += __builtin_amdgcn_readlane(ic, kWave - 1);
      ba += __popcll(lead);
    }
    Span sp = make_span(lo, hi, A, k, c_lo, c_hi, NB);
    if (sp.e0 < 0 && sp.a0 < A) {   // the start rolled over to the next expert
      sp.e0 = C.ex_id[sp.a0];
      sp.n0 = C.ex_n[sp.a0];
    }
    if (lane == 0) {
      C.ex_row[A] = tnu & 0xFFFF;
      C.ex_unit[A] = tnu >> 16;
      C.ex_cost[A] = tc;
      L.nA[0] = A;
      L.span[0] = sp.a0; L.span[1] = sp.g0; L.span[2] = sp.s0; L.span[3] = sp.e0;
      L.span[4] = sp.n0; L.span[5] = sp.rb0; L.span[6] = sp.left; L.span[7] = sp.row_limit;
    }
  }
  __syncthreads();
  C.A = uni(L.nA[0]);
}

// Pair mode, for small batches (T*k <= kPairMax): every (token, expert) pair is its own
// unit of one token, in pair order, so every step of every unit costs the same and the
// workgroup's span is closed-form (no table build); the first unit's expert is one
// scalar load of topk_ids. An expert named by several tokens is read once per token (at
// decode sizes a few percent more bytes). Entries outside [0, E) read expert 0 (their
// outputs are unspecified).
__device__ __forceinline__ Span pair_span(const ExpertArgs& a, const ClassCost& k, float inv_steps, int NB, int b,
                                          int G) {
  const int steps = k.steps;
  (void)G;
  int l0, len;
  split_at(b, a.pn1, a.pq1, a.pr1, a.pq2, a.pr2, l0, len);
  const int l1 = l0 + len;
  Span sp;
  sp.a0 = div_by(l0, inv_steps);
  sp.s0 = l0 - sp.a0 * steps;
  sp.g0 = 0;
  sp.n0 = 1;
  sp.rb0 = sp.a0;
  sp.left = (l1 - l0) * NB;
  const int a1 = div_by(l1, inv_steps);
  sp.row_limit = a1 + (l1 - a1 * steps > 0 ? 1 : 0);
  sp.e0 = 0;
  return sp;
}

__device__ __forceinline__ Span read_span(const ExpertLds& L) {
  Span sp;
  sp.a0 = uni(L.span[0]); sp.g0 = uni(L.span[1]); sp.s0 = uni(L.span[2]); sp.e0 = uni(L.span[3]);
  sp.n0 = uni(L.span[4]); sp.rb0 = uni(L.span[5]); sp.left = uni(L.span[6]); sp.row_limit = uni(L.span[7]);
  return sp;
}

// Routed class rows: each pair's token goes to its expert's rows at the rank of the
// token among the expert's tokens (a token naming one expert twice keeps one row).
// Ends with an LDS barrier.
__device__ __forceinline__ void build_rows(const ExpertArgs& a, const ExpertLds& L, const ClassTab& C) {
  const int P = a.T * a.k;
  for (int p = threadIdx.x; p < P; p += kBlock) {
    const int e = L.ids[p];
    if ((unsigned)e < (unsigned)a.E) {
      const int t = p / a.k;
      const int r = L.ebase[e] + tok_rank(L, e, t);
      C.r_tok[r] = t;
      C.r_pair[r] = p;
      C.r_exp[r] = e;
    }
  }
  lds_barrier();
}

// Where the current unit's data sits: its first class row, its first staged row, its
// token count, its expert and the pair index of each of its rows.
struct UnitCtx {
  int crow, wrow, n, e;
  int pr[4];
  float g[2];   // GEMV walks: the expert's global weight scales (gate/up: gate, up; down: [0])
};

// How a walk reads its class: units (expert, token count, first row), the unit count, and
// each class row's token and pair index.
//   VW_TAB     routed experts from the LDS tables (build_routed / build_rows)
//   VW_PAIR    pair mode: unit a is pair a (one token, row a), its expert from topk_ids
//              staged in LDS (entries outside [0, E) read expert 0)
//   VW_SHARED  the shared expert: one unit of all T tokens, row t = token t
enum { VW_TAB = 0, VW_PAIR = 1, VW_SHARED = 2 };
template <int VW>
struct ClassView {
  const ClassTab* C;
  const int* lids;
  int k, E, T, P;
  float inv_k;   // 1 / k: token r / k of pair row r as (r + 1/2) / k in FP32, exact for r < 2^16
  __device__ __forceinline__ int count() const {
    if constexpr (VW == VW_TAB) return C->A;
    else if constexpr (VW == VW_PAIR) return P;
    else return 1;
  }
  __device__ __forceinline__ void unit(int a, int& e, int& n, int& rb) const {
    if constexpr (VW == VW_TAB) {
      e = uni(C->ex_id[a]); n = uni(C->ex_n[a]); rb = uni(C->ex_row[a]);
    } else if constexpr (VW == VW_PAIR) {
      const int v = uni(lids[a]);
      e = (unsigned)v < (unsigned)E ? v : 0; n = 1; rb = a;
    } else {
      e = 0; n = T; rb = 0;
    }
  }
  __device__ __forceinline__ int tok(int r) const {
    if constexpr (VW == VW_TAB) return C->r_tok[r];
    else if constexpr (VW == VW_PAIR) return (int)(((float)r + 0.5f) * inv_k);
    else return r;
  }
  __device__ __forceinline__ int pair(int r) const {
    if constexpr (VW == VW_TAB) return C->r_pair[r];
    else if constexpr (VW == VW_PAIR) return r;
    else return P + r;
  }
};

constexpr int kGsPer = 8;   // narrow token items: global weight scales staged per thread (2 E <= 8 kBlock)

// Routing fused into the gate/up walk (pair mode): where the router logits are and where
// the selection goes (logits == nullptr: not fused).
struct FusedRoute {
  const float* logits;
  int32_t* ids_out;
  float* w_out;
  int E, k;
  float inv_k;
  const float* raw;        // bare logits [T][E] when the bias only selects, or NULL
  int softmax;             // combine weights from the softmax (1) or the sigmoid (0)
};

// Walks one workgroup's span of a class. The class's operations (workgroup-uniform):
//   op.rows(e, s, lrow, out[RPL])  global weight rows of this lane at step s of expert e
//   op.ld(tok, pair, el) -> uint4  raw bytes behind 16 staged bytes of a row at element el
//   op.cv(uint4) -> uint4          those 16 staged bytes
//   op.tsc(tok, pair) -> float     a row's activation scale
//   op.sink(ctx, s, lrow, acc)     results, on the lanes with jl == 0 (the unit's global
//                                  weight scales in ctx.g: scalar loads at each unit
//                                  change, whose latency the step's weight wait hides)
// Ops is a plain struct per (projection, activation format), so the shared and routed
// classes run the same code whenever their formats agree.
// Prologue: the first staged window (rows of the first units, which the span alone
// names) and, in pair mode, topk_ids are loaded into registers; then the first weight loads are issued (they
// need only the first unit's expert, sp.e0); then everything goes to LDS. So the weights
// are in flight one memory round trip after launch. Two register sets alternate (no
// loop-carried copy); every step but the last issues the same number of weight loads for
// the next one, so the compiler waits for one step's loads while the next step's are in
// flight. Later windows are staged when a unit does not fit; only LDS barriers are used,
// so weight loads stream across them.
template <int FMT, int AK, int RPL, int VW, int NKF, bool FRAW, class Ops>
__device__ __forceinline__ void walk_class(const WTensor& W, const GemvMap& m, const ExpertLds& L,
                                           int lds_tile_bytes, const ClassView<VW>& V, const ClassCost& k,
                                           const Span& sp, const Ops& op, const int32_t* ids,
                                           const FusedRoute fr = FusedRoute{}) {
  constexpr int EPL = elems_per_piece(FMT);
  constexpr int PER = AK == 0 ? 8 : 4;
  if (sp.left <= 0) return;
  int left = sp.left;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int jl = lane & (m.LPR - 1), lrow = wave * m.G + (lane >> m.lg);
  const int tstride = W.K * m.esize;
  const int cap = m.cap;
  const int A = V.count();
  // NVFP4: the wave's staged scales (1 KB of LDS per wave after the tile)
  const ScaleChunk sk = FMT == W_NVFP4 ? scale_chunk<FMT, RPL>(m, W.scale_row_bytes) : ScaleChunk{0, 0, 0, 0, 0};
  uint8_t* const sca = L.tile + lds_tile_bytes + wave * kScaleStageWave;
  auto advance = [&](Cursor& p) {
    if (++p.b < m.NB) return;
    p.b = 0;
    if (++p.s < k.steps) return;
    p.s = 0;
    if (++p.g * k.NG < p.n) return;
    p.g = 0;
    if (++p.a < A) V.unit(p.a, p.e, p.n, p.rb);
  };
  auto row_ld = [&](int r0) {
    return [&, r0](int t, int el) { return op.ld(V.tok(r0 + t), V.pair(r0 + t), el); };
  };
  int r0 = sp.rb0 + sp.g0 * k.NG;   // staged class rows [r0, r1)
  constexpr int NS = RPL == 2 ? kPreSlotsGateup : kPreSlots;   // prologue register slots
  int r1 = min(min(r0 + cap, sp.row_limit), r0 + m.win);
  auto stage = [&](int ra) {
    lds_barrier();                  // everyone is done with the previous rows
    r0 = ra;
    r1 = min(ra + cap, sp.row_limit);
    const int nrows = r1 - r0;
    stage_tile<AK, EPL>(L.tile, m, W.K, nrows, row_ld(r0), [&](uint4 r) { return op.cv(r); });
    for (int i = threadIdx.x; i < nrows; i += kBlock) L.w_tsc[i] = op.tsc(V.tok(r0 + i), V.pair(r0 + i));
    lds_barrier();
  };
  float acc[RPL][4];
  int cur_a = -1, cur_g = -1;
  UnitCtx cx{0, 0, 0, 0, {0, 0, 0, 0}, {1.0f, 1.0f}};
  auto do_step = [&](auto pf, const Cursor& p, WeightRegs<RPL>& cur, WeightRegs<RPL>& nxt, Cursor& np) {
    if (p.a != cur_a || p.g != cur_g) {   // next unit
      cur_a = p.a;
      cur_g = p.g;
      const int ur = p.rb + p.g * k.NG;
      const int nt = min(k.NG, p.n - p.g * k.NG);
      if (ur + nt > r1) stage(ur);
      cx.crow = ur;
      cx.wrow = ur - r0;
      cx.n = nt;
      cx.e = p.e;
#pragma unroll
      for (int t = 0; t < 4; ++t) cx.pr[t] = t < nt ? V.pair(ur + t) : 0;
      // (every load issues: without gscale it reads the first codes and takes 1)
      const float* gp = W.gscale ? W.gscale + (int64_t)p.e * W.gs_per_expert : reinterpret_cast<const float*>(W.codes);
#pragma unroll
      for (int q = 0; q < RPL; ++q) {
        const float gv = reinterpret_cast<const __attribute__((address_space(4))) float*>((uintptr_t)gp)[W.gscale ? q : 0];
        cx.g[q] = W.gscale ? gv : 1.0f;
      }
    }
    if (p.b == 0) {
#pragma unroll
      for (int q = 0; q < RPL; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[q][t] = 0.0f;
    }
    if constexpr (decltype(pf)::value) {
      np = p;
      advance(np);
      int64_t nr[RPL];
      op.rows(np.e, np.s, lrow, nr);
      fetch_batch<FMT, RPL>(W, m, nr, np.b, jl, sk, nxt);
    }
    const uint8_t* tile = L.tile + cx.wrow * tstride;
    const int n = VW == VW_PAIR ? 1 : cx.n;   // a pair is one token
    if constexpr (FMT == W_NVFP4) *reinterpret_cast<uint4*>(sca + lane * 16) = cur.sc;   // (the batch's scales)
#pragma unroll
    for (int i = 0; i < WeightRegs<RPL>::NPB; ++i) {
      if (i < m.NPB) {
        const int pc = p.b * m.NPB + i;
        uint32_t sv[RPL];
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
          if constexpr (FMT == W_NVFP4)
            sv[q] = *reinterpret_cast<const uint16_t*>(sca + q * sk.qbytes + (lane >> m.lg) * sk.bb +
                                                       (((i * m.LPR + jl) * EPL) >> 4));
          else
            sv[q] = cur.s[i][q];
        }
        // the empty asm statements keep the three variants real (scalar) branches: with
        // nothing but arithmetic in them the compiler would run all three and select
        if (n == 1) {
          asm volatile("");
          accumulate_piece<FMT, AK, 1, RPL>(cur.w[i], sv, tile, tstride, m.LPR, pc, jl, acc);
        } else if (AK == 1 || n == 2) {
          asm volatile("");
          accumulate_piece<FMT, AK, 2, RPL>(cur.w[i], sv, tile, tstride, m.LPR, pc, jl, acc);
        } else {
          asm volatile("");
          accumulate_piece<FMT, AK, 4, RPL>(cur.w[i], sv, tile, tstride, m.LPR, pc, jl, acc);
        }
      }
    }
    if (p.b == m.NB - 1) {
#pragma unroll
      for (int q = 0; q < RPL; ++q)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if (t < n) {
            float v = acc[q][t];
            for (int o = m.LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
            acc[q][t] = v;
          }
        }
      if (jl == 0) op.sink(cx, p.s, lrow, acc);
    }
  };
  // prologue: loads that need no expert id, then the first weight loads, then LDS. With
  // fused routing (NKF > 0 slots per lane, pair mode) the router logits of the span's
  // tokens are loaded first and the experts are selected while the other prologue loads
  // are in flight.
  constexpr bool FUSED = VW == VW_PAIR && NKF > 0;
  constexpr int NKL = NKF > 0 ? NKF : 1;
  const int nrows0 = r1 - r0;
  struct NoTopk {};
  std::conditional_t<FUSED, TopkIn<NKL, FRAW>, NoTopk> lv;   // (nothing without fused routing)
  int t_lo = 0, t_hi = -1;
  auto route_load = [&](int t) {
    if constexpr (FUSED) {
      const int64_t off = (int64_t)min(t, t_hi) * fr.E;
      wave_topk_load<NKL, FRAW>(fr.logits + off, FRAW ? fr.raw + off : nullptr, fr.E, lv);
    }
  };
  if constexpr (FUSED) {
    t_lo = div_by(sp.a0, fr.inv_k);
    t_hi = div_by(sp.row_limit - 1, fr.inv_k);
    route_load(t_lo + wave);
  }
  uint4 raw[NS];
  const SlotMap<AK> smap(m, W.K);
  park_rows<AK, NS>(smap, nrows0, row_ld(r0), raw);
  float ts_r = 0.0f;
  if ((int)threadIdx.x < nrows0) ts_r = op.tsc(V.tok(r0 + threadIdx.x), V.pair(r0 + threadIdx.x));
  int idv = 0;
  if constexpr (VW == VW_PAIR) {
    if (ids) idv = ids[min((int)threadIdx.x, V.P - 1)];
  }
  Cursor pa{sp.a0, sp.g0, sp.s0, 0, sp.e0, sp.n0, sp.rb0}, pb = pa;
  if constexpr (FUSED) {   // one token per wave (more rounds for longer spans), then the first expert
    for (int tb = t_lo; tb <= t_hi; tb += kBlock / kWave) {
      const int t = tb + wave;
      if (tb != t_lo) route_load(t);
      int e;
      float w;
      wave_topk_select<NKL, FRAW>(lv, fr.E, fr.k, fr.softmax, e, w);
      if (t <= t_hi && lane < fr.k) {
        L.ids[t * fr.k + lane] = e;
        fr.ids_out[t * fr.k + lane] = e;
        fr.w_out[t * fr.k + lane] = w;
      }
    }
    lds_barrier();
    const int e0 = uni(L.ids[sp.a0]);
    pa.e = (unsigned)e0 < (unsigned)fr.E ? e0 : 0;
  }
  WeightRegs<RPL> A_, B_;
  {
    int64_t rr[RPL];
    op.rows(pa.e, pa.s, lrow, rr);
    fetch_batch<FMT, RPL>(W, m, rr, 0, jl, sk, A_);
  }
  unpark_rows<AK, EPL, NS>(smap, L.tile, nrows0, [&](uint4 r) { return op.cv(r); }, raw);
  if ((int)threadIdx.x < nrows0) L.w_tsc[threadIdx.x] = ts_r;
  if constexpr (VW == VW_PAIR) {
    if (ids && (int)threadIdx.x < V.P) L.ids[threadIdx.x] = idv;
  }
  lds_barrier();
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  while (true) {
    if (left == 1) { do_step(No{}, pa, A_, B_, pb); break; }
    do_step(Yes{}, pa, A_, B_, pb);
    if (left == 2) { do_step(No{}, pb, B_, A_, pa); break; }
    do_step(Yes{}, pb, B_, A_, pa);
    left -= 2;
  }
}

// Activation slot sources, in two halves so that the loads can be issued long before
// the LDS stores: a load returns the raw bytes behind 16 bytes of staged activations
// (8 BF16 or 4 FP32 values) at element el, a convert turns them into those 16 bytes.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint4 cv_same(uint4 r) { return r; }
// NVFP4: 8 codes (4 bytes) and their E4M3 block scale; converted to 8 BF16 (v * S, exact).
__device__ __forceinline__ uint4 nvfp4_ld(const uint8_t* codes, const uint8_t* scales, int el) {
  return make_uint4(*reinterpret_cast<const uint32_t*>(codes + (el >> 1)), scales[el >> 4], 0u, 0u);
}
__device__ __forceinline__ uint4 nvfp4_cv(uint4 r) {
  const float S = e4m3_to_f32(r.y);
  const uint32_t w = r.x;
  uint32_t o[4];
  const f32x2_t v0 = fp4x2_to_f32<0>(w, 1.0f), v1 = fp4x2_to_f32<1>(w, 1.0f);
  const f32x2_t v2 = fp4x2_to_f32<2>(w, 1.0f), v3 = fp4x2_to_f32<3>(w, 1.0f);
  o[0] = (__float_as_uint(v0.x * S) >> 16) | (__float_as_uint(v0.y * S) & 0xFFFF0000u);
  o[1] = (__float_as_uint(v1.x * S) >> 16) | (__float_as_uint(v1.y * S) & 0xFFFF0000u);
  o[2] = (__float_as_uint(v2.x * S) >> 16) | (__float_as_uint(v2.y * S) & 0xFFFF0000u);
  o[3] = (__float_as_uint(v3.x * S) >> 16) | (__float_as_uint(v3.y * S) & 0xFFFF0000u);
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// FP8-E4M3: 8 codes; converted to 8 BF16 (exact).
__device__ __forceinline__ uint4 fp8_ld(const uint8_t* codes, int el) {
  const uint2 w = *reinterpret_cast<const uint2*>(codes + el);
  return make_uint4(w.x, w.y, 0u, 0u);
}
__device__ __forceinline__ uint4 fp8_cv(uint4 r) {
  return make_uint4(as_u32(fp8x2_to_bf16<false>(r.x, 1.0f)), as_u32(fp8x2_to_bf16<true>(r.x, 1.0f)),
                    as_u32(fp8x2_to_bf16<false>(r.y, 1.0f)), as_u32(fp8x2_to_bf16<true>(r.y, 1.0f)));
}

// MXFP4: 8 E2M1 codes (4 bytes) and their block's E8M0 scale; converted to 8 BF16
// (v * 2^e, exact: E2M1 values times a power of two fit BF16 down to its subnormals).
__device__ __forceinline__ uint4 mxfp4_ld(const uint8_t* codes, const uint8_t* scales, int el) {
  return make_uint4(*reinterpret_cast<const uint32_t*>(codes + (el >> 1)), scales[el >> 5], 0u, 0u);
}
__device__ __forceinline__ uint4 mxfp4_cv(uint4 r) {
  const float sc = e8m0_to_f32(r.y);
  return make_uint4(as_u32(fp4x2_to_bf16<0>(r.x, sc)), as_u32(fp4x2_to_bf16<1>(r.x, sc)),
                    as_u32(fp4x2_to_bf16<2>(r.x, sc)), as_u32(fp4x2_to_bf16<3>(r.x, sc)));
}
// MXFP8: 8 E4M3 codes and their block's E8M0 scale; converted to 8 BF16 (exact but for
// E4M3 subnormals scaled below BF16's smallest subnormal, 2^-133).
__device__ __forceinline__ uint4 mxfp8_ld(const uint8_t* codes, const uint8_t* scales, int el) {
  const uint2 w = *reinterpret_cast<const uint2*>(codes + el);
  return make_uint4(w.x, w.y, scales[el >> 5], 0u);
}
__device__ __forceinline__ uint4 mxfp8_cv(uint4 r) {
  const float sc = e8m0_to_f32(r.z);
  return make_uint4(as_u32(fp8x2_to_bf16<false>(r.x, sc)), as_u32(fp8x2_to_bf16<true>(r.x, sc)),
                    as_u32(fp8x2_to_bf16<false>(r.y, sc)), as_u32(fp8x2_to_bf16<true>(r.y, sc)));
}

// ================================================================ gate/up kernel
// Gate/up rows: at row-step s, lane row slot lrow is intermediate index
// i = s * PS + lrow (PS = 4 * G pairs per step); the lane holds gate row i (q = 0) and
// up row I + i (q = 1). AF is the format the class's activations arrive in.
template <int AF>
struct GateupOps {
  const uint16_t* x;
  const uint8_t* xq_codes;
  const uint8_t* xq_scales;
  const float* xq_scale;
  const float* gscale;
  int gs_per_expert, wrows, Iexp, PS, H, hs;
  float* h;
  float* dbg_h;
  const float* w_tsc;
  const int* r_pair;
  int h_bf16;            // GEMV kernels: store h as BF16 (RNE) for the down GEMV

  __device__ __forceinline__ void rows(int e, int st, int lrow, int64_t (&out)[2]) const {
    const int64_t base = (int64_t)e * wrows;
    const int i = st * PS + lrow;
    out[0] = base + i;
    out[1] = base + Iexp + i;
  }
  __device__ __forceinline__ uint4 ld(int t, int, int el) const {
    if constexpr (AF == A_NVFP4_4O6)
      return nvfp4_ld(xq_codes + (int64_t)t * (H / 2), xq_scales + (int64_t)t * (H / 16), el);
    else if constexpr (AF == A_FP8_TOKEN)
      return fp8_ld(xq_codes + (int64_t)t * H, el);
    else if constexpr (AF == A_MXFP4)
      return mxfp4_ld(xq_codes + (int64_t)t * (H / 2), xq_scales + (int64_t)t * (H / 32), el);
    else if constexpr (AF == A_MXFP8)
      return mxfp8_ld(xq_codes + (int64_t)t * H, xq_scales + (int64_t)t * (H / 32), el);
    else
      return ld16(x + (int64_t)t * H + el);
  }
  __device__ __forceinline__ uint4 cv(uint4 r) const {
    if constexpr (AF == A_NVFP4_4O6) return nvfp4_cv(r);
    else if constexpr (AF == A_FP8_TOKEN) return fp8_cv(r);
    else if constexpr (AF == A_MXFP4) return mxfp4_cv(r);
    else if constexpr (AF == A_MXFP8) return mxfp8_cv(r);
    else return r;
  }
  __device__ __forceinline__ float tsc(int t, int) const { return afmt_row_scaled(AF) ? xq_scale[t] : 1.0f; }
  // the raw code bytes and E8M0 scales of token t's row (scaled-MFMA staging)
  __device__ __forceinline__ const uint8_t* codes_row(int t, int) const {
    return xq_codes + (int64_t)t * (AF == A_MXFP4 ? H / 2 : H);
  }
  __device__ __forceinline__ const uint8_t* scales_row(int t, int) const { return xq_scales + (int64_t)t * (H / 32); }
  __device__ __forceinline__ float gs(int e, int q) const {
    return gscale ? gscale[(int64_t)e * gs_per_expert + q] : 1.0f;
  }
  __device__ __forceinline__ void sink(const UnitCtx& cx, int st, int lrow, const float (&acc)[2][4]) const {
    const int i = st * PS + lrow;
    const float gsg = cx.g[0], gsu = cx.g[1];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < cx.n) {
        const float ts = w_tsc[cx.wrow + t];
        const float gv = acc[0][t] * gsg * ts;
        const float uv = acc[1][t] * gsu * ts;
        const float hv = gv / (1.0f + expf(-gv)) * uv;
        const int64_t off = (int64_t)cx.pr[t] * hs + i;
        // a BF16 row keeps the byte position of its FP32 row (rows of both kinds share h)
        if (h_bf16) reinterpret_cast<uint16_t*>(h)[off + (int64_t)cx.pr[t] * hs] = (uint16_t)f32_to_bf16_rne(hv);
        else h[off] = hv;
        if (dbg_h) dbg_h[off] = hv;
      }
    }
  }
};

__device__ __forceinline__ ClassCost gateup_cost(const ExpertArgs& a, bool routed) {
  const GemvMap& m = routed ? a.rmap : a.smap;
  return ClassCost{m.NG, m.steps, m.cw, m.ct};
}

template <int VW>
__device__ __forceinline__ ClassView<VW> class_view(const ExpertArgs& a, const ExpertLds& L) {
  return ClassView<VW>{&L.rt, L.ids, a.k, a.E, a.T, a.T * a.k, a.inv_k};
}

template <int FMT, int AF, int VW, int NKF = 0, bool FRAW = false>
__device__ __forceinline__ void gateup_walk(const ExpertArgs& a, const ExpertLds& L, const Span& sp,
                                            const int32_t* ids, const FusedRoute fr = FusedRoute{}) {
  constexpr bool routed = VW != VW_SHARED;
  const WTensor& W = routed ? a.rw : a.sw;
  const GemvMap& m = routed ? a.rmap : a.smap;
  const int Iexp = routed ? a.I : a.Ish;
  const GateupOps<AF> op{a.x, a.xq_codes, a.xq_scales, a.xq_scale, W.gscale, W.gs_per_expert, W.rows, Iexp,
                         4 * m.G, a.H, a.hs, a.h, a.dbg_h, L.w_tsc, nullptr, AF == A_BF16};
  walk_class<FMT, 0, 2, VW, NKF, FRAW>(W, m, L, a.lds_act_bytes, class_view<VW>(a, L), gateup_cost(a, routed), sp, op,
                                 ids, fr);
}

// How a GEMV launch walks the routed experts (the same for every workgroup of a launch,
// so each is a kernel of its own: a kernel's registers are sized for the largest path it
// holds, and the table builds need far more than the pair and token walks).
enum { RW_PAIR = 0, RW_TABLE = 1, RW_TOKEN = 2, RW_TOKEN_WIDE = 3 };

// Workgroups [0, sh_wgs) walk the shared expert (BF16 activations, no dependency on the
// routing), the others split the selected experts: pairs (MODE = RW_PAIR, a.pair_mode)
// or the tables' units (RW_TABLE). NKF > 0 (pair mode, a.fuse_topk): the walk's prologue
// selects the experts from the router logits, NKF = fused_topk_slots(E) slots per lane;
// FRAW: with bare logits (a router bias that only selects, a.raw != NULL).
template <int RF, int SF, int AF, int MODE, int NKF, bool FRAW = false>
__global__ void __launch_bounds__(kBlock, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) gateup_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  warm_args<ExpertArgs>();
  ExpertLds L = carve(a, smem);
  const bool shared = (int)blockIdx.x < a.sh_wgs;
  if (shared) {
    const Span sp = shared_span(a.T, gateup_cost(a, false), a.smap.NB, blockIdx.x, a.sh_wgs,
                                ShareW{0, a.ncu, a.late16});
    gateup_walk<SF, A_BF16, VW_SHARED>(a, L, sp, nullptr);
  } else if constexpr (MODE == RW_PAIR) {
    Span sp = pair_span(a, gateup_cost(a, true), a.rmap.inv_steps, a.rmap.NB, blockIdx.x - a.sh_wgs,
                        gridDim.x - a.sh_wgs);
    if constexpr (NKF > 0) {   // (a workgroup with an empty span selects nothing)
      const FusedRoute fr{a.logits, a.ids_out, a.w_out, a.E, a.k, a.inv_k, a.raw, a.softmax};
      gateup_walk<RF, AF, VW_PAIR, NKF, FRAW>(a, L, sp, nullptr, fr);
    } else {
      if (sp.a0 < a.T * a.k) {
        const int e = a.ids[sp.a0];
        sp.e0 = (unsigned)e < (unsigned)a.E ? e : 0;
      }
      gateup_walk<RF, AF, VW_PAIR>(a, L, sp, a.ids);
    }
  } else {
    build_routed(a, L, L.rt, gateup_cost(a, true), a.rmap.NB, blockIdx.x - a.sh_wgs, gridDim.x - a.sh_wgs);
    build_rows(a, L, L.rt);
    gateup_walk<RF, AF, VW_TAB>(a, L, read_span(L), nullptr);
  }
}

// =================================================================== down kernel
// Writes each (pair, hidden row) partial output o, scaled by the weight's global scale
// and the pair's activation scale; the combine kernel sums them. Each lane holds one row
// (RPL = 1): at row-step s, lane row slot lrow is hidden row s * RS + lrow. AF is the
// routed experts' activation format: h is staged as FP32 for BF16 (and for the shared
// expert), as BF16 values decoded from the re-quantized h otherwise.
template <int AF>
struct DownOps {
  const float* hf;
  const uint8_t* hq_codes;
  const uint8_t* hq_scales;
  const float* hq_scale;
  const float* gscale;
  int gs_per_expert, wrows, Kexp, RS, H, hs;
  float* o;
  const float* w_tsc;
  const int* r_pair;
  int h_bf16;            // h stored as BF16 (GEMV kernels)

  __device__ __forceinline__ void rows(int e, int st, int lrow, int64_t (&out)[1]) const {
    out[0] = (int64_t)e * wrows + st * RS + lrow;
  }
  __device__ __forceinline__ uint4 ld(int, int p, int el) const {
    if constexpr (AF == A_NVFP4_4O6)
      return nvfp4_ld(hq_codes + (int64_t)p * (Kexp / 2), hq_scales + (int64_t)p * (Kexp / 16), el);
    else if constexpr (AF == A_FP8_TOKEN)
      return fp8_ld(hq_codes + (int64_t)p * Kexp, el);
    else if constexpr (AF == A_MXFP4)
      return mxfp4_ld(hq_codes + (int64_t)p * (Kexp / 2), hq_scales + (int64_t)p * (Kexp / 32), el);
    else if constexpr (AF == A_MXFP8)
      return mxfp8_ld(hq_codes + (int64_t)p * Kexp, hq_scales + (int64_t)p * (Kexp / 32), el);
    else if (h_bf16)   // BF16 rows at the byte positions of FP32 rows
      return ld16(reinterpret_cast<const uint16_t*>(hf) + (int64_t)p * (2 * hs) + el);
    else
      return ld16(hf + (int64_t)p * hs + el);
  }
  __device__ __forceinline__ uint4 cv(uint4 r) const {
    if constexpr (AF == A_NVFP4_4O6) return nvfp4_cv(r);
    else if constexpr (AF == A_FP8_TOKEN) return fp8_cv(r);
    else if constexpr (AF == A_MXFP4) return mxfp4_cv(r);
    else if constexpr (AF == A_MXFP8) return mxfp8_cv(r);
    else return r;
  }
  __device__ __forceinline__ float tsc(int, int p) const { return afmt_row_scaled(AF) ? hq_scale[p] : 1.0f; }
  // the raw code bytes and E8M0 scales of pair p's h row (scaled-MFMA staging)
  __device__ __forceinline__ const uint8_t* codes_row(int, int p) const {
    return hq_codes + (int64_t)p * (AF == A_MXFP4 ? Kexp / 2 : Kexp);
  }
  __device__ __forceinline__ const uint8_t* scales_row(int, int p) const {
    return hq_scales + (int64_t)p * (Kexp / 32);
  }
  __device__ __forceinline__ float gs(int e, int q) const {
    return (q == 0 && gscale) ? gscale[(int64_t)e * gs_per_expert] : 1.0f;
  }
  __device__ __forceinline__ void sink(const UnitCtx& cx, int st, int lrow, const float (&acc)[1][4]) const {
    const float g = cx.g[0];
    const int row = st * RS + lrow;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      if (t < cx.n) o[(int64_t)cx.pr[t] * H + row] = acc[0][t] * g * w_tsc[cx.wrow + t];
  }
};

__device__ __forceinline__ ClassCost down_cost(const ExpertArgs& a, bool routed) {
  const GemvMap& m = routed ? a.rmap : a.smap;
  return ClassCost{m.NG, m.steps, m.cw, m.ct};
}

template <int FMT, int AF, int VW>
__device__ __forceinline__ void down_walk(const ExpertArgs& a, const ExpertLds& L, const Span& sp) {
  constexpr bool routed = VW != VW_SHARED;
  const WTensor& W = routed ? a.rw : a.sw;
  const GemvMap& m = routed ? a.rmap : a.smap;
  const DownOps<AF> op{a.h, a.hq_codes, a.hq_scales, a.hq_scale, W.gscale, W.gs_per_expert, W.rows,
                       routed ? a.I : a.Ish, m.RS, a.H, a.hs, a.o, L.w_tsc, nullptr, 1};
  walk_class<FMT, 0, 1, VW, 0, false>(W, m, L, a.lds_act_bytes, class_view<VW>(a, L), down_cost(a, routed), sp, op,
                               a.ids);
}

// Token mode of the down projection (pair mode, when the shared expert, if any, has the
// routed format and size and takes the same FP32 h): a work item is (token t, row-step
// s), i.e. a block of hidden rows of y[t]; its J = k (+1 shared) sub-steps are the
// token's experts. Each sub-step's dot products are scaled by its combine weight, global
// weight scale and activation scale and summed in registers; the item writes the BF16
// sum to y: the weighted combine needs no per-pair output. Items split evenly over the
// workgroups. The J activation rows of the current token sit in LDS (rows j of the
// tile); the first token's are loaded before the first weight loads, as in walk_class.
//   WIDE = false: an item is RS = 4 G rows, each wave G of them over all J sub-steps (all
//     of an item's weight loads are issued at once: kTokJMax register sets of kTokPieces
//     pieces, one memory round trip per item).
//   WIDE = true: an item is G rows and the waves split the sub-steps (wave w takes j = w
//     and w + 4), so a batch of few tokens still has enough items to fill the GPU; the
//     four waves' partial sums meet in LDS and are added in wave order.
template <int FMT, int AK, int AF, bool WIDE>
__device__ __forceinline__ void walk_tokens(const ExpertArgs& a, const ExpertLds& L, int i0, int i1) {
  constexpr int EPL = elems_per_piece(FMT);
  constexpr int NPT = kTokPieces;
  constexpr int NJ = WIDE ? kTokJMax / 4 : kTokJMax;   // sub-steps per lane
  if (i1 <= i0) return;
  const GemvMap& m = a.rmap;
  const int items = a.tok_items, J = a.k + a.has_shared, P = a.T * a.k;
  const int lane = threadIdx.x & (kWave - 1), wave = uni((int)threadIdx.x / kWave);
  const int jl = lane & (m.LPR - 1), lrow = (WIDE ? 0 : wave * m.G) + (lane >> m.lg);
  const int rows_item = WIDE ? m.G : m.RS;
  const int tstride = a.rw.K * m.esize;
  auto jof = [&](int jj) { return WIDE ? wave + 4 * jj : jj; };
  const DownOps<AF> op{a.h, a.hq_codes, a.hq_scales, a.hq_scale, a.rw.gscale, a.rw.gs_per_expert, a.rw.rows,
                       a.I, m.RS, a.H, a.hs, a.o, L.w_tsc, nullptr, 1};
  auto pair_of = [&](int t, int j) { return j < a.k ? t * a.k + j : P + t; };
  auto clamp_e = [&](int v) { return (unsigned)v < (unsigned)a.E ? v : 0; };
  struct Regs {
    uint4 w[NPT];
    uint32_t s[NPT];
    float g;   // WIDE, routed sub-steps: the expert's global weight scale (1 without one)
  };
  // sub-step j of item row-step s of token t, expert e: this lane's NPT pieces of its row.
  // WIDE (two sub-steps per lane) also loads a routed expert's global scale as a scalar
  // load (e is wave-uniform) instead of staging every expert's scales; with the narrow
  // items' eight sub-steps per lane those scalars would spill.
  auto fetch = [&](int s, int j, int e, Regs& R) {
    const bool sh = j >= a.k;
    if constexpr (WIDE) {
      const float* gp = a.rw.gscale ? a.rw.gscale + (int64_t)e * a.rw.gs_per_expert
                                    : reinterpret_cast<const float*>(a.rw.codes);
      const float gv = *(const __attribute__((address_space(4))) float*)(uintptr_t)gp;
      R.g = a.rw.gscale ? gv : 1.0f;
    }
    const uint8_t* codes = sh ? a.sw.codes : a.rw.codes;
    const uint8_t* scales = sh ? a.sw.scales : a.rw.scales;
    const int64_t row = (int64_t)(sh ? 0 : e) * a.rw.rows + s * rows_item + lrow;
    const uint8_t* rp = codes + row * a.rw.code_row_bytes;
    const uint8_t* sp = scales ? scales + row * a.rw.scale_row_bytes : nullptr;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int el = (min(i, m.NPB - 1) * m.LPR + jl) * EPL;
      R.w[i] = load_stream16(rp + elem_byte<FMT>(el));
      if constexpr (FMT == W_NVFP4)
        R.s[i] = *reinterpret_cast<const uint16_t*>(sp + (el >> 4));
      else if constexpr (FMT == W_MXFP4 || FMT == W_MXFP8)
        R.s[i] = sp[el >> 5];
      else
        R.s[i] = 0u;
    }
  };
  auto row_ld = [&](int t) {
    return [&, t](int j, int el) { return op.ld(t, pair_of(t, j), el); };
  };
  // per-row factor: combine weight (1 for the shared row) times activation scale
  auto row_fac = [&](int t, int j) {
    const int p = pair_of(t, j);
    return op.tsc(t, p) * (j < a.k ? a.topk_w[p] : 1.0f);
  };
  int staged_t = div_by(i0, a.tok_inv);
  auto stage = [&](int t) {
    lds_barrier();
    stage_tile<AK, EPL>(L.tile, m, a.rw.K, J, row_ld(t), [&](uint4 r) { return op.cv(r); });
    if ((int)threadIdx.x < J) L.w_tsc[threadIdx.x] = row_fac(t, threadIdx.x);
    staged_t = t;
    lds_barrier();
  };
  float* red = L.w_gs;   // WIDE: [4][G] partial sums of the waves
  // one item from the weight registers R (experts ex) of its sub-steps
  auto item = [&](int it, const Regs (&R)[NJ], const int (&ex)[NJ]) {
    const int t = div_by(it, a.tok_inv), s = it - t * items;
    float tot = 0.0f;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = jof(jj);
      if (j < J) {
        float part[1][4];
        part[0][0] = 0.0f;
        const uint8_t* tile = L.tile + j * tstride;
        WeightRegs<1> wr;
#pragma unroll
        for (int i = 0; i < WeightRegs<1>::NPB; ++i) {
          wr.w[i][0] = R[jj].w[min(i, NPT - 1)];
          wr.s[i][0] = R[jj].s[min(i, NPT - 1)];
        }
#pragma unroll
        for (int i = 0; i < NPT; ++i)
          if (i < m.NPB) accumulate_piece<FMT, AK, 1, 1>(wr.w[i], wr.s[i], tile, tstride, m.LPR, i, jl, part);
        const float g = j >= a.k ? L.gs_sh[0] : (WIDE ? R[jj].g : L.gs_rt[ex[jj] * a.rw.gs_per_expert]);
        tot = fmaf(L.w_tsc[j] * g, part[0][0], tot);
      }
    }
    for (int o = m.LPR / 2; o > 0; o >>= 1) tot += __shfl_xor(tot, o, kWave);
    if constexpr (WIDE) {
      lds_barrier();   // the previous item's partial sums have been read
      if (jl == 0) red[wave * m.G + lrow] = tot;
      lds_barrier();
      if ((int)threadIdx.x < m.G) {
        const int r = threadIdx.x;
        const int64_t yi = (int64_t)t * a.H + s * rows_item + r;
        float v = ((red[r] + red[m.G + r]) + red[2 * m.G + r]) + red[3 * m.G + r];
        if (a.resid) v += bf16_to_f32(a.resid[yi]);   // the residual add, then one rounding
        a.y[yi] = (uint16_t)f32_to_bf16_rne(v);
      }
    } else {
      if (jl == 0) {
        const int64_t yi = (int64_t)t * a.H + s * rows_item + lrow;
        if (a.resid) tot += bf16_to_f32(a.resid[yi]);
        a.y[yi] = (uint16_t)f32_to_bf16_rne(tot);
      }
    }
  };
  // the weight loads of item `it` (its experts from the staged topk_ids)
  auto fetch_item = [&](int it, Regs (&R)[NJ], int (&ex)[NJ]) {
    const int t = div_by(it, a.tok_inv);
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int j = jof(jj);
      if (j < J) {
        ex[jj] = j < a.k ? clamp_e(uni(L.ids[t * a.k + j])) : 0;
        fetch(it - t * items, j, ex[jj], R[jj]);
      }
    }
  };
  Regs RA[NJ], RB[NJ];
  int exA[NJ], exB[NJ];
  // prologue: the first token's experts (scalar loads), rows, factors, global scales
  // (narrow: every routed expert's; wide: the shared expert's) and topk_ids, then every
  // sub-step's weight loads (wide: and routed global scales) of the first item, then LDS
#pragma unroll
  for (int jj = 0; jj < NJ; ++jj) {   // every load issued (clamped index), so they go out as one batch
    const int j = jof(jj);
    const int v = a.ids[staged_t * a.k + min(j, a.k - 1)];
    exA[jj] = j < a.k && j < J ? clamp_e(v) : 0;
  }
  uint4 raw[kPreSlotsTok];
  const SlotMap<AK> smap(m, a.rw.K);
  park_rows<AK, kPreSlotsTok>(smap, J, row_ld(staged_t), raw);
  const float fac_r = row_fac(staged_t, min((int)threadIdx.x, J - 1));
  // narrow items: every routed expert's global scale, staged in LDS
  constexpr int NGS = WIDE ? 1 : kGsPer;
  const int ngs = a.E * a.rw.gs_per_expert;
  const float* gsrc = a.rw.gscale ? a.rw.gscale : reinterpret_cast<const float*>(a.rw.codes);
  const int gmax = a.rw.gscale ? ngs - 1 : 0;
  float gsv[NGS];
  if constexpr (!WIDE) {
#pragma unroll
    for (int j = 0; j < NGS; ++j) gsv[j] = gsrc[min((int)threadIdx.x + j * kBlock, gmax)];
  }
  const float* ssrc = a.sw.gscale ? a.sw.gscale : reinterpret_cast<const float*>(a.sw.codes);
  const float gss = ssrc[0];
  const int idv = a.ids[min((int)threadIdx.x, P - 1)];
  {
    const int s0 = i0 - staged_t * items;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
      if (jof(jj) < J) fetch(s0, jof(jj), exA[jj], RA[jj]);
  }
  unpark_rows<AK, EPL, kPreSlotsTok>(smap, L.tile, J, [&](uint4 r) { return op.cv(r); }, raw);
  if ((int)threadIdx.x < J) L.w_tsc[threadIdx.x] = fac_r;
  if constexpr (!WIDE) {
#pragma unroll
    for (int j = 0; j < NGS; ++j) {
      const int i = threadIdx.x + j * kBlock;
      if (i < ngs) L.gs_rt[i] = a.rw.gscale ? gsv[j] : 1.0f;
    }
  }
  if (threadIdx.x == 0) L.gs_sh[0] = a.sw.gscale ? gss : 1.0f;
  if ((int)threadIdx.x < P) L.ids[threadIdx.x] = idv;
  lds_barrier();
  if constexpr (WIDE) {
    // two register sets alternate: the next item's weight loads are in flight while
    // this item computes (a token change restages the rows after this item)
    int it = i0;
    auto step = [&](auto pf, const Regs (&Rc)[NJ], const int (&exc)[NJ], Regs (&Rn)[NJ], int (&exn)[NJ]) {
      if constexpr (decltype(pf)::value) fetch_item(it + 1, Rn, exn);
      item(it, Rc, exc);
      ++it;
      if constexpr (decltype(pf)::value) {
        const int t = div_by(it, a.tok_inv);
        if (t != staged_t) stage(t);
      }
    };
    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    while (true) {
      if (i1 - it == 1) { step(No{}, RA, exA, RB, exB); break; }
      step(Yes{}, RA, exA, RB, exB);
      if (i1 - it == 1) { step(No{}, RB, exB, RA, exA); break; }
      step(Yes{}, RB, exB, RA, exA);
    }
  } else {
    item(i0, RA, exA);
    for (int it = i0 + 1; it < i1; ++it) {
      const int t = div_by(it, a.tok_inv);
      if (t != staged_t) stage(t);
      fetch_item(it, RA, exA);
      item(it, RA, exA);
    }
  }
}

// MODE: RW_TOKEN or RW_TOKEN_WIDE (a.token_mode 1 or 2: token items over all of a
// token's experts, writing y; the shared expert, if any, has the routed format), else the
// shared expert's workgroups and the routed pairs (RW_PAIR) or tables' units (RW_TABLE),
// as in gate/up.
template <int RF, int SF, int AF, int MODE>
__global__ void __launch_bounds__(kBlock, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) down_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  warm_args<ExpertArgs>();
  ExpertLds L = carve(a, smem);
  if constexpr (MODE == RW_TOKEN || MODE == RW_TOKEN_WIDE) {
    static_assert(SF == RF, "token mode reads the shared expert as a routed one");
    int i0, len;   // items per workgroup: the host's two-round split
    split_at(blockIdx.x, a.pn1, a.pq1, a.pr1, a.pq2, a.pr2, i0, len);
    walk_tokens<RF, 0, AF, MODE == RW_TOKEN_WIDE>(a, L, i0, i0 + len);
    return;
  }
  const bool shared = (int)blockIdx.x < a.sh_wgs;
  if (shared) {
    const Span sp = shared_span(a.T, down_cost(a, false), a.smap.NB, blockIdx.x, a.sh_wgs,
                                ShareW{0, a.ncu, a.late16});
    down_walk<SF, A_BF16, VW_SHARED>(a, L, sp);
  } else if constexpr (MODE == RW_PAIR) {
    Span sp = pair_span(a, down_cost(a, true), a.rmap.inv_steps, a.rmap.NB, blockIdx.x - a.sh_wgs,
                        gridDim.x - a.sh_wgs);
    if (sp.a0 < a.T * a.k) {
      const int e = a.ids[sp.a0];
      sp.e0 = (unsigned)e < (unsigned)a.E ? e : 0;
    }
    down_walk<RF, AF, VW_PAIR>(a, L, sp);
  } else {
    build_routed(a, L, L.rt, down_cost(a, true), a.rmap.NB, blockIdx.x - a.sh_wgs, gridDim.x - a.sh_wgs);
    build_rows(a, L, L.rt);
    down_walk<RF, AF, VW_TAB>(a, L, read_span(L));
  }
}

// ================================================================ host launchers
hipError_t launch_hquant(const ExpertArgs& a, hipStream_t s);
hipError_t launch_combine(const ExpertArgs& a, hipStream_t s);

// gate/up -> (h re-quantization) -> down -> combine, in stream order.
template <int RF, int SF, int AF>
__global__ void ggateup_kernel(ExpertArgs a);
template <int RF, int SF, int AF>
__global__ void gdown_kernel(ExpertArgs a);

template <int RF, int SF, int AF>
hipError_t launch_experts_af(const ExpertArgs& gu, int gu_grid, size_t gu_lds,
                             const ExpertArgs& dn, int dn_grid, size_t dn_lds, hipStream_t s) {
  auto go = [&](int kind, auto kern, int grid, size_t lds, const ExpertArgs& a) {
    return launch_kernel(kind, kern, dim3(grid), dim3(kBlock), lds, s, a);
  };
  const int nkf = gu.fuse_topk ? fused_topk_slots(gu.E) : 0;
  const bool fraw = gu.raw != nullptr;
  hipError_t err = gu.grouped     ? go(K_GATEUP, ggateup_kernel<RF, SF, AF>, gu_grid, gu_lds, gu)
                   : !gu.pair_mode ? go(K_GATEUP, gateup_kernel<RF, SF, AF, RW_TABLE, 0>, gu_grid, gu_lds, gu)
                   : nkf == 0     ? go(K_GATEUP, gateup_kernel<RF, SF, AF, RW_PAIR, 0>, gu_grid, gu_lds, gu)
                   : nkf == 2 ? (fraw ? go(K_GATEUP, gateup_kernel<RF, SF, AF, RW_PAIR, 2, true>, gu_grid, gu_lds, gu)
                                      : go(K_GATEUP, gateup_kernel<RF, SF, AF, RW_PAIR, 2>, gu_grid, gu_lds, gu))
                   : nkf == 4 ? (fraw ? go(K_GATEUP, gateup_kernel<RF, SF, AF, RW_PAIR, 4, true>, gu_grid, gu_lds, gu)
                                      : go(K_GATEUP, gateup_kernel<RF, SF, AF, RW_PAIR, 4>, gu_grid, gu_lds, gu))
                   : fraw ? go(K_GATEUP, gateup_kernel<RF, SF, AF, RW_PAIR, 8, true>, gu_grid, gu_lds, gu)
                          : go(K_GATEUP, gateup_kernel<RF, SF, AF, RW_PAIR, 8>, gu_grid, gu_lds, gu);
  if (err != hipSuccess) return err;
  if (AF != A_BF16 && (err = launch_hquant(gu, s)) != hipSuccess) return err;
  if (dn.grouped) {
    err = go(K_DOWN, gdown_kernel<RF, SF, AF>, dn_grid, dn_lds, dn);
  } else if (dn.token_mode) {
    if constexpr (SF == RF) {
      err = dn.token_mode == 2 ? go(K_DOWN, down_kernel<RF, SF, AF, RW_TOKEN_WIDE>, dn_grid, dn_lds, dn)
                               : go(K_DOWN, down_kernel<RF, SF, AF, RW_TOKEN>, dn_grid, dn_lds, dn);
    } else {
      return hipErrorInvalidValue;   // the plan never picks token mode for a shared expert of another format
    }
  } else {
    err = dn.pair_mode ? go(K_DOWN, down_kernel<RF, SF, AF, RW_PAIR>, dn_grid, dn_lds, dn)
                       : go(K_DOWN, down_kernel<RF, SF, AF, RW_TABLE>, dn_grid, dn_lds, dn);
  }
  if (err != hipSuccess) return err;
  return dn.token_mode ? hipSuccess : launch_combine(dn, s);
}

// The activation formats each routed weight format supports (the ABI checks refuse the
// other pairs before any launch).
template <int RF, int SF>
hipError_t launch_experts_t(const ExpertArgs& gu, int gu_grid, size_t gu_lds,
                            const ExpertArgs& dn, int dn_grid, size_t dn_lds, hipStream_t s) {
  if (gu.afmt == A_BF16) return launch_experts_af<RF, SF, A_BF16>(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, s);
  if constexpr (RF == W_NVFP4) {
    if (gu.afmt == A_NVFP4_4O6)
      return launch_experts_af<RF, SF, A_NVFP4_4O6>(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, s);
  }
  if constexpr (RF == W_MXFP4 || RF == W_MXFP8) {
    if (gu.afmt == A_FP8_TOKEN)
      return launch_experts_af<RF, SF, A_FP8_TOKEN>(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, s);
    if (gu.afmt == A_MXFP4)
      return launch_experts_af<RF, SF, A_MXFP4>(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, s);
    if (gu.afmt == A_MXFP8)
      return launch_experts_af<RF, SF, A_MXFP8>(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
