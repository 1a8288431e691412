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
  uint64_t* tmask;  // [E] token mask of each expert
  int* ebase;       // [E] first routed class row of each selected expert
  int* ids;         // [T*k] topk_ids
  int* nA;          // [4] selected expert count
  ClassTab rt, sh;
  float* w_gs;      // [2 * kWinRows] global weight scales of the staged rows' experts
  float* w_tsc;     // [kWinRows] activation scales of the staged rows
  uint8_t* tile;    // activations of the staged rows, K * esize bytes each
};

__device__ __forceinline__ ExpertLds carve(const ExpertArgs& a, uint8_t* smem) {
  ExpertLds L;
  const int P = a.T * a.k, Am = min(a.E, P);
  L.tmask = reinterpret_cast<uint64_t*>(smem);
  L.ebase = reinterpret_cast<int*>(L.tmask + a.E);
  L.ids = L.ebase + a.E;
  L.nA = L.ids + P;
  int* q = L.nA + 4;
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
  L.tile = smem + a.lds_list_bytes;
  return L;
}

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

// The routed class from topk_ids (synchronizes): token masks, then wave 0 compacts the
// selected experts in id order (ballots) and scans their tokens, units and costs.
// Entries outside [0, E) are ignored. Class rows are filled later by build_rows.
__device__ __forceinline__ void build_routed(const ExpertArgs& a, const ExpertLds& L, ClassTab& C, int NG,
                                             int steps, int cw, int ct) {
  const int P = a.T * a.k;
  for (int i = threadIdx.x; i < a.E; i += kBlock) L.tmask[i] = 0ull;
  __syncthreads();
  for (int p = threadIdx.x; p < P; p += kBlock) {
    const int e = a.ids[p];
    L.ids[p] = e;
    if ((unsigned)e < (unsigned)a.E)
      atomicOr(reinterpret_cast<unsigned long long*>(&L.tmask[e]), 1ull << (p / a.k));
  }
  __syncthreads();
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const uint64_t below = (1ull << lane) - 1ull;
    int A = 0;
    for (int c0 = 0; c0 < a.E; c0 += kWave) {
      const int e = c0 + lane;
      const int n = e < a.E ? __popcll(L.tmask[e]) : 0;
      const uint64_t bal = __ballot(n > 0);
      if (n > 0) {
        const int i = A + __popcll(bal & below);
        C.ex_id[i] = e;
        C.ex_n[i] = n;
      }
      A += __popcll(bal);
    }
    int rr = 0, ru = 0, rc = 0;
    for (int c0 = 0; c0 < A; c0 += kWave) {
      const int i = c0 + lane;
      const int n = i < A ? C.ex_n[i] : 0;
      const int u = (n + NG - 1) / NG;
      const int c = steps * (cw * u + ct * n);
      int xn = n, xu = u, xc = c;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const int yn = __shfl_up(xn, off, kWave), yu = __shfl_up(xu, off, kWave);
        const int yc = __shfl_up(xc, off, kWave);
        if (lane >= off) { xn += yn; xu += yu; xc += yc; }
      }
      if (i < A) {
        C.ex_row[i] = rr + xn - n;
        C.ex_unit[i] = ru + xu - u;
        C.ex_cost[i] = rc + xc - c;
        L.ebase[C.ex_id[i]] = rr + xn - n;
      }
      rr += __shfl(xn, kWave - 1, kWave);
      ru += __shfl(xu, kWave - 1, kWave);
      rc += __shfl(xc, kWave - 1, kWave);
    }
    if (lane == 0) {
      C.ex_row[A] = rr;
      C.ex_unit[A] = ru;
      C.ex_cost[A] = rc;
      L.nA[0] = A;
    }
  }
  __syncthreads();
  C.A = uni(L.nA[0]);
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
      const int r = L.ebase[e] + __popcll(L.tmask[e] & ((1ull << t) - 1ull));
      C.r_tok[r] = t;
      C.r_pair[r] = p;
      C.r_exp[r] = e;
    }
  }
  lds_barrier();
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

// Stage all K elements of nt tokens into the LDS tile.
//   AK = 0: BF16 values (exact), 8 per slot;  AK = 1: FP32 values, 4 per slot.
// src(t, el) returns the 16-byte slot for token t at element el.
template <int AK, int EPL, class Src>
__device__ __forceinline__ void stage_tile(uint8_t* tile, const GemvMap& m, int K, int nt, Src src) {
  constexpr int PER = AK == 0 ? 8 : 4;
  constexpr int NSUB = EPL / PER;
  const int units = K / PER;
  const int tstride = K * m.esize;
  for (int u = threadIdx.x; u < nt * units; u += kBlock) {
    const int t = u / units, el = (u % units) * PER;
    const int pc = el / EPL, sub = (el % EPL) / PER;
    *reinterpret_cast<uint4*>(tile + t * tstride + act_slot(pc, sub, NSUB, m.LPR)) = src(t, el);
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
          const uint8_t* p = base + t * tstride;
          const uint4 a0 = *reinterpret_cast<const uint4*>(p);
          const uint4 a1 = *reinterpret_cast<const uint4*>(p + sstride);
          const uint4 a2 = *reinterpret_cast<const uint4*>(p + 2 * sstride);
          const uint4 a3 = *reinterpret_cast<const uint4*>(p + 3 * sstride);
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
          const uint8_t* p = base + t * tstride;
          const uint4 a0 = *reinterpret_cast<const uint4*>(p);
          const uint4 a1 = *reinterpret_cast<const uint4*>(p + sstride);
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
          const uint4 a0 = *reinterpret_cast<const uint4*>(base + t * tstride);
          float r = acc[q][t];
          r = dot2(w[0], a0.x, r); r = dot2(w[1], a0.y, r);
          r = dot2(w[2], a0.z, r); r = dot2(w[3], a0.w, r);
          acc[q][t] = r;
        }
      }
    } else {  // FP32 activations
      if constexpr (FMT == W_NVFP4 || FMT == W_MXFP4) {
        const float sc = FMT == W_MXFP4 ? e8m0_to_f32(sv[q] & 0xFFu) : 1.0f;
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
            const uint8_t* p = base + t * tstride + 4 * half * sstride;
            float pp = 0.0f;
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
              const float4 av = *reinterpret_cast<const float4*>(p + sb * sstride);
              pp = fmaf(wf[4 * sb + 0], av.x, pp);
              pp = fmaf(wf[4 * sb + 1], av.y, pp);
              pp = fmaf(wf[4 * sb + 2], av.z, pp);
              pp = fmaf(wf[4 * sb + 3], av.w, pp);
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
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const uint8_t* p = base + t * tstride;
          float r = acc[q][t];
#pragma unroll
          for (int sb = 0; sb < 4; ++sb) {
            const float4 av = *reinterpret_cast<const float4*>(p + sb * sstride);
            r = fmaf(wf[4 * sb + 0], av.x, r); r = fmaf(wf[4 * sb + 1], av.y, r);
            r = fmaf(wf[4 * sb + 2], av.z, r); r = fmaf(wf[4 * sb + 3], av.w, r);
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
};

// Loads batch b (pieces b*NPB .. b*NPB + NPB - 1) of the lane's rows. Always issues
// exactly NPB_max x RPL weight loads and as many scale loads (slots beyond the batch
// reload its first piece): a step-independent count lets the compiler wait for one
// step's loads while the next step's are still in flight (vector-memory counters
// retire in issue order).
template <int FMT, int RPL>
__device__ __forceinline__ void fetch_batch(const WTensor& W, const GemvMap& m, const int64_t (&rows)[RPL],
                                            int b, int jl, WeightRegs<RPL>& R) {
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
      if constexpr (FMT == W_NVFP4)
        R.s[i][q] = *reinterpret_cast<const uint16_t*>(sp + (el >> 4));
      else if constexpr (FMT == W_MXFP4 || FMT == W_MXFP8)
        R.s[i][q] = sp[el >> 5];
      else
        R.s[i][q] = 0u;
    }
  }
}

// ===================================================================== work walk
// A walk position: batch b of row-step s of group g of the class's expert index a
// (expert id e with n tokens, first class row rb).
struct Cursor {
  int a, g, s, b;
  int e, n, rb;
};

// Cost parameters of one class in one kernel.
struct ClassCost {
  int NG, steps, cw, ct;
};

// First position (b = 0) whose start cost is >= c; a == A when c >= the class total.
// Workgroup-uniform.
__device__ __forceinline__ void pos_at(const ClassTab& C, const ClassCost& k, int c, int& a, int& g, int& s) {
  const int lane = threadIdx.x & (kWave - 1);
  int cnt = 0;
  for (int c0 = 0; c0 < C.A; c0 += kWave) {
    const int i = c0 + lane;
    cnt += __popcll(__ballot(i < C.A && C.ex_cost[i] <= c));
  }
  g = 0; s = 0;
  if (c >= uni(C.ex_cost[C.A])) { a = C.A; return; }
  a = cnt - 1;
  const int n = uni(C.ex_n[a]);
  const int G = (n + k.NG - 1) / k.NG;
  const int rem = c - uni(C.ex_cost[a]);
  const int F = k.steps * (k.cw + k.ct * k.NG);
  g = min(rem / F, G - 1);
  const int cs = k.cw + k.ct * min(k.NG, n - g * k.NG);
  s = (rem - g * F + cs - 1) / cs;
  if (s >= k.steps) {
    s = 0;
    if (++g >= G) { g = 0; ++a; }
  }
}

// Where the current unit's data sits: its first class row, its first staged row, and
// its token count.
struct UnitCtx {
  int crow, wrow, n;
};

// Walks the positions of one class whose start cost lies in [c_lo, c_hi).
// Call-backs (workgroup-uniform):
//   rows(e, s, lrow, out[RPL])     global weight rows of this lane at step s of expert e
//   prep()                         runs once after the first weight loads are issued,
//                                  before the first staging (ends with a barrier)
//   src(tok, pair, el) -> uint4    16 bytes of a row's activations at element el
//   tsc(tok, pair) -> float        a row's activation scale
//   gs(e, q) -> float              global weight scale q of expert e
//   sink(ctx, s, lrow, acc)        results, on the lanes with jl == 0
// Two register sets alternate (no loop-carried copy); every step but the last issues
// the same number of weight loads for the next one, so the compiler waits for one
// step's loads while the next step's are in flight (vector-memory counters retire in
// issue order). Staged rows are a window of consecutive class rows, restaged only when
// a unit does not fit; only LDS barriers are used, so weight loads stream across it.
template <int FMT, int AK, int RPL, class Rows, class Prep, class Src, class Tsc, class Gs, class Sink>
__device__ __forceinline__ void walk_class(const WTensor& W, const GemvMap& m, const ExpertLds& L,
                                           int lds_tile_bytes, const ClassTab& C, const ClassCost& k,
                                           int c_lo, int c_hi, Rows rows, Prep prep, Src src, Tsc tsc,
                                           Gs gs, Sink sink) {
  constexpr int EPL = elems_per_piece(FMT);
  int a0, g0, s0, a1, g1, s1;
  pos_at(C, k, c_lo, a0, g0, s0);
  pos_at(C, k, c_hi, a1, g1, s1);
  const int l0 = (uni(C.ex_unit[a0]) + g0) * k.steps + s0;
  const int l1 = (uni(C.ex_unit[a1]) + g1) * k.steps + s1;
  if (l1 <= l0) return;
  int left = (l1 - l0) * m.NB;   // positions to walk
  // one past the last class row walked
  int row_limit = uni(C.ex_row[a1]) + g1 * k.NG;
  if (s1 > 0) row_limit += min(k.NG, uni(C.ex_n[a1]) - g1 * k.NG);

  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int jl = lane % m.LPR, lrow = wave * m.G + lane / m.LPR;
  const int tstride = W.K * m.esize;
  const int cap = min(kWinRows, lds_tile_bytes / tstride);
  auto advance = [&](Cursor& p) {
    if (++p.b < m.NB) return;
    p.b = 0;
    if (++p.s < k.steps) return;
    p.s = 0;
    if (++p.g * k.NG < p.n) return;
    p.g = 0;
    if (++p.a < C.A) {
      p.e = uni(C.ex_id[p.a]);
      p.n = uni(C.ex_n[p.a]);
      p.rb = uni(C.ex_row[p.a]);
    }
  };
  int r0 = 0, r1 = 0;            // staged class rows [r0, r1)
  int cur_a = -1, cur_g = -1;
  UnitCtx cx{0, 0, 0};
  auto stage = [&](int ra) {
    lds_barrier();               // everyone is done with the previous rows
    r0 = ra;
    r1 = min(ra + cap, row_limit);
    const int nrows = r1 - r0;
    stage_tile<AK, EPL>(L.tile, m, W.K, nrows, [&](int r, int el) {
      return src(C.r_tok[r0 + r], C.r_pair[r0 + r], el);
    });
    for (int i = threadIdx.x; i < nrows; i += kBlock) {
      const int tk = C.r_tok[r0 + i], pr = C.r_pair[r0 + i], e = C.r_exp[r0 + i];
      L.w_tsc[i] = tsc(tk, pr);
      L.w_gs[2 * i] = gs(e, 0);
      L.w_gs[2 * i + 1] = gs(e, 1);
    }
    lds_barrier();
  };
  float acc[RPL][4];
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
      rows(np.e, np.s, lrow, nr);
      fetch_batch<FMT, RPL>(W, m, nr, np.b, jl, nxt);
    }
    const uint8_t* tile = L.tile + cx.wrow * tstride;
    const int n = cx.n;
#pragma unroll
    for (int i = 0; i < WeightRegs<RPL>::NPB; ++i) {
      if (i < m.NPB) {
        const int pc = p.b * m.NPB + i;
        // the empty asm statements keep the three variants real (scalar) branches: with
        // nothing but arithmetic in them the compiler would run all three and select
        if (n == 1) {
          asm volatile("");
          accumulate_piece<FMT, AK, 1, RPL>(cur.w[i], cur.s[i], tile, tstride, m.LPR, pc, jl, acc);
        } else if (AK == 1 || n == 2) {
          asm volatile("");
          accumulate_piece<FMT, AK, 2, RPL>(cur.w[i], cur.s[i], tile, tstride, m.LPR, pc, jl, acc);
        } else {
          asm volatile("");
          accumulate_piece<FMT, AK, 4, RPL>(cur.w[i], cur.s[i], tile, tstride, m.LPR, pc, jl, acc);
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
      if (jl == 0) sink(cx, p.s, lrow, acc);
    }
  };
  Cursor pa{a0, g0, s0, 0, uni(C.ex_id[a0]), uni(C.ex_n[a0]), uni(C.ex_row[a0])}, pb = pa;
  WeightRegs<RPL> A, B;
  {
    int64_t rr[RPL];
    rows(pa.e, pa.s, lrow, rr);
    fetch_batch<FMT, RPL>(W, m, rr, 0, jl, A);
  }
  prep();
  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  while (true) {
    if (left == 1) { do_step(No{}, pa, A, B, pb); break; }
    do_step(Yes{}, pa, A, B, pb);
    if (left == 2) { do_step(No{}, pb, B, A, pa); break; }
    do_step(Yes{}, pb, B, A, pa);
    left -= 2;
  }
}

// This workgroup's share [c_lo, c_hi) of the summed cost of both classes.
__device__ __forceinline__ void wg_share(int total, int& c_lo, int& c_hi) {
  c_lo = (int)((long long)total * blockIdx.x / gridDim.x);
  c_hi = (int)((long long)total * (blockIdx.x + 1) / gridDim.x);
}

// Activation slot sources. Each returns 16 bytes: 8 BF16 values or 4 FP32 values.
__device__ __forceinline__ uint4 bf16_slot(const uint16_t* row, int el) {
  return *reinterpret_cast<const uint4*>(row + el);
}
// 8 NVFP4 values -> 8 BF16 (v * S, exact in BF16).
__device__ __forceinline__ uint4 nvfp4_slot(const uint8_t* codes, const uint8_t* scales, int el) {
  const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + (el >> 1));
  const float S = e4m3_to_f32(scales[el >> 4]);
  uint32_t o[4];
  const f32x2_t v0 = fp4x2_to_f32<0>(w, 1.0f), v1 = fp4x2_to_f32<1>(w, 1.0f);
  const f32x2_t v2 = fp4x2_to_f32<2>(w, 1.0f), v3 = fp4x2_to_f32<3>(w, 1.0f);
  o[0] = (__float_as_uint(v0.x * S) >> 16) | (__float_as_uint(v0.y * S) & 0xFFFF0000u);
  o[1] = (__float_as_uint(v1.x * S) >> 16) | (__float_as_uint(v1.y * S) & 0xFFFF0000u);
  o[2] = (__float_as_uint(v2.x * S) >> 16) | (__float_as_uint(v2.y * S) & 0xFFFF0000u);
  o[3] = (__float_as_uint(v3.x * S) >> 16) | (__float_as_uint(v3.y * S) & 0xFFFF0000u);
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// 8 FP8-E4M3 values -> 8 BF16 (exact).
__device__ __forceinline__ uint4 fp8_slot(const uint8_t* codes, int el) {
  const uint2 w = *reinterpret_cast<const uint2*>(codes + el);
  return make_uint4(as_u32(fp8x2_to_bf16<false>(w.x, 1.0f)), as_u32(fp8x2_to_bf16<true>(w.x, 1.0f)),
                    as_u32(fp8x2_to_bf16<false>(w.y, 1.0f)), as_u32(fp8x2_to_bf16<true>(w.y, 1.0f)));
}
__device__ __forceinline__ uint4 f32_slot(const float* row, int el) {
  return *reinterpret_cast<const uint4*>(row + el);
}

// ================================================================ gate/up kernel
// Gate/up rows: at row-step s, lane row slot lrow is intermediate index
// i = s * PS + lrow (PS = 4 * G pairs per step); the lane holds gate row i (q = 0) and
// up row I + i (q = 1).
template <int FMT, class Prep>
__device__ __forceinline__ void gateup_walk(const ExpertArgs& a, const ExpertLds& L, const ClassTab& C,
                                            bool routed, int c_lo, int c_hi, Prep prep) {
  const WTensor& W = routed ? a.rw : a.sw;
  const GemvMap& m = routed ? a.rmap : a.smap;
  const int PS = 4 * m.G;
  const int Iexp = routed ? a.I : a.Ish;
  const int afmt = routed ? a.afmt : A_BF16;
  const ClassCost k{m.NG, Iexp / PS, m.cw, m.ct};
  auto rows = [&](int e, int st, int lrow, int64_t (&out)[2]) {
    const int64_t base = (int64_t)e * W.rows;
    const int i = st * PS + lrow;
    out[0] = base + i;
    out[1] = base + Iexp + i;
  };
  auto tsc = [&](int t, int) { return afmt == A_BF16 ? 1.0f : a.xq_scale[t]; };
  auto gs = [&](int e, int q) { return W.gscale ? W.gscale[(int64_t)e * W.gs_per_expert + q] : 1.0f; };
  auto sink = [&](const UnitCtx& cx, int st, int lrow, const float (&acc)[2][4]) {
    const int i = st * PS + lrow;
    const float gsg = L.w_gs[2 * cx.wrow], gsu = L.w_gs[2 * cx.wrow + 1];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < cx.n) {
        const float ts = L.w_tsc[cx.wrow + t];
        const float gv = acc[0][t] * gsg * ts;
        const float uv = acc[1][t] * gsu * ts;
        const float hv = gv / (1.0f + expf(-gv)) * uv;
        const int64_t off = (int64_t)C.r_pair[cx.crow + t] * a.hs + i;
        a.h[off] = hv;
        if (a.dbg_h) a.dbg_h[off] = hv;
      }
    }
  };
  if (afmt == A_NVFP4_4O6) {
    walk_class<FMT, 0, 2>(W, m, L, a.lds_act_bytes, C, k, c_lo, c_hi, rows, prep,
        [&](int t, int, int el) {
          return nvfp4_slot(a.xq_codes + (int64_t)t * (a.H / 2), a.xq_scales + (int64_t)t * (a.H / 16), el);
        }, tsc, gs, sink);
  } else if (afmt == A_FP8_TOKEN) {
    walk_class<FMT, 0, 2>(W, m, L, a.lds_act_bytes, C, k, c_lo, c_hi, rows, prep,
        [&](int t, int, int el) { return fp8_slot(a.xq_codes + (int64_t)t * a.H, el); }, tsc, gs, sink);
  } else {
    walk_class<FMT, 0, 2>(W, m, L, a.lds_act_bytes, C, k, c_lo, c_hi, rows, prep,
        [&](int t, int, int el) { return bf16_slot(a.x + (int64_t)t * a.H, el); }, tsc, gs, sink);
  }
}

template <int RF, int SF>
__global__ void __launch_bounds__(kBlock, 2) gateup_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  ExpertLds L = carve(a, smem);
  if (a.has_shared) build_shared(a, L.sh, a.smap.NG, a.Ish / (4 * a.smap.G), a.smap.cw, a.smap.ct);
  build_routed(a, L, L.rt, a.rmap.NG, a.I / (4 * a.rmap.G), a.rmap.cw, a.rmap.ct);
  const int cs = a.has_shared ? uni(L.sh.ex_cost[1]) : 0;
  int c_lo, c_hi;
  wg_share(cs + uni(L.rt.ex_cost[L.rt.A]), c_lo, c_hi);
  if (c_lo < cs) gateup_walk<SF>(a, L, L.sh, false, c_lo, min(c_hi, cs), [] {});
  if (c_hi > cs)
    gateup_walk<RF>(a, L, L.rt, true, max(c_lo - cs, 0), c_hi - cs, [&] { build_rows(a, L, L.rt); });
}

// =================================================================== down kernel
// Writes each (pair, hidden row) partial output o, scaled by the weight's global scale
// and the pair's activation scale; the combine kernel sums them. Each lane holds one row
// (RPL = 1): at row-step s, lane row slot lrow is hidden row s * RS + lrow.
template <int FMT, int AK, int RPL, class Prep>
__device__ __forceinline__ void down_walk(const ExpertArgs& a, const ExpertLds& L, const ClassTab& C,
                                          bool routed, int c_lo, int c_hi, Prep prep) {
  const WTensor& W = routed ? a.rw : a.sw;
  const GemvMap& m = routed ? a.rmap : a.smap;
  const int RS = m.RS;
  const int Kexp = routed ? a.I : a.Ish;
  const int afmt = routed ? a.afmt : A_BF16;
  const ClassCost k{m.NG, a.H / RS, m.cw, m.ct};
  auto rows = [&](int e, int st, int lrow, int64_t (&out)[RPL]) {
    const int64_t base = (int64_t)e * W.rows + st * RS + lrow * RPL;
#pragma unroll
    for (int q = 0; q < RPL; ++q) out[q] = base + q;
  };
  auto tsc = [&](int, int p) { return afmt == A_BF16 ? 1.0f : a.hq_scale[p]; };
  auto gs = [&](int e, int q) {
    return (q == 0 && W.gscale) ? W.gscale[(int64_t)e * W.gs_per_expert] : 1.0f;
  };
  auto sink = [&](const UnitCtx& cx, int st, int lrow, const float (&acc)[RPL][4]) {
    const float g = L.w_gs[2 * cx.wrow];
    const int row0 = st * RS + lrow * RPL;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < cx.n) {
        const float sc = g * L.w_tsc[cx.wrow + t];
        float* o = a.o + (int64_t)C.r_pair[cx.crow + t] * a.H + row0;
#pragma unroll
        for (int q = 0; q < RPL; ++q) o[q] = acc[q][t] * sc;
      }
    }
  };
  if constexpr (AK == 1) {
    walk_class<FMT, 1, RPL>(W, m, L, a.lds_act_bytes, C, k, c_lo, c_hi, rows, prep,
        [&](int, int p, int el) { return f32_slot(a.h + (int64_t)p * a.hs, el); }, tsc, gs, sink);
  } else if (afmt == A_NVFP4_4O6) {
    walk_class<FMT, 0, RPL>(W, m, L, a.lds_act_bytes, C, k, c_lo, c_hi, rows, prep,
        [&](int, int p, int el) {
          return nvfp4_slot(a.hq_codes + (int64_t)p * (Kexp / 2), a.hq_scales + (int64_t)p * (Kexp / 16), el);
        }, tsc, gs, sink);
  } else {
    walk_class<FMT, 0, RPL>(W, m, L, a.lds_act_bytes, C, k, c_lo, c_hi, rows, prep,
        [&](int, int p, int el) { return fp8_slot(a.hq_codes + (int64_t)p * Kexp, el); }, tsc, gs, sink);
  }
}


template <int RF, int SF, int RAK>
__global__ void __launch_bounds__(kBlock, 2) down_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  ExpertLds L = carve(a, smem);
  if (a.has_shared) build_shared(a, L.sh, a.smap.NG, a.H / a.smap.RS, a.smap.cw, a.smap.ct);
  build_routed(a, L, L.rt, a.rmap.NG, a.H / a.rmap.RS, a.rmap.cw, a.rmap.ct);
  const int cs = a.has_shared ? uni(L.sh.ex_cost[1]) : 0;
  int c_lo, c_hi;
  wg_share(cs + uni(L.rt.ex_cost[L.rt.A]), c_lo, c_hi);
  if (c_lo < cs) down_walk<SF, 1, 1>(a, L, L.sh, false, c_lo, min(c_hi, cs), [] {});
  if (c_hi > cs)
    down_walk<RF, RAK, 1>(a, L, L.rt, true, max(c_lo - cs, 0), c_hi - cs, [&] { build_rows(a, L, L.rt); });
}

// ================================================================ host launchers
hipError_t launch_hquant(const ExpertArgs& a, hipStream_t s);
hipError_t launch_combine(const ExpertArgs& a, hipStream_t s);

// gate/up -> (h re-quantization) -> down -> combine, in stream order.
template <int RF, int SF>
hipError_t launch_experts_t(const ExpertArgs& gu, int gu_grid, size_t gu_lds,
                            const ExpertArgs& dn, int dn_grid, size_t dn_lds, hipStream_t s) {
  hipError_t err = launch_kernel(K_GATEUP, gateup_kernel<RF, SF>, dim3(gu_grid), dim3(kBlock), gu_lds, s, gu);
  if (err != hipSuccess) return err;
  if (gu.afmt != A_BF16 && (err = launch_hquant(gu, s)) != hipSuccess) return err;
  err = dn.afmt == A_BF16
      ? launch_kernel(K_DOWN, down_kernel<RF, SF, 1>, dim3(dn_grid), dim3(kBlock), dn_lds, s, dn)
      : launch_kernel(K_DOWN, down_kernel<RF, SF, 0>, dim3(dn_grid), dim3(kBlock), dn_lds, s, dn);
  if (err != hipSuccess) return err;
  return launch_combine(dn, s);
}

}  // namespace moe
