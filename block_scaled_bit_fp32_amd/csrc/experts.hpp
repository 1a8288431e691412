// Dequant-fused expert GEMVs for gfx950: gate/up with SwiGLU, down with the combine.
//
//   gateup_kernel  one workgroup per (selected expert, chunk of intermediate rows) plus
//                  (shared expert, chunk); gate and up rows of the same chunk, SwiGLU in
//                  the epilogue; the last workgroup of each routed expert re-quantizes
//                  that expert's h rows when the layer quantizes h.
//   down_kernel    one workgroup per (selected expert, chunk of hidden rows); the last
//                  workgroup of each hidden chunk combines every expert's partial output
//                  in a fixed order and writes BF16 y.
// Each workgroup streams its weight rows once with 16-byte loads, decodes them in
// registers (gfx950 FP4/FP8 converts) and takes activations from an LDS tile.
// "Last workgroup" hand-offs use a device-scope counter after a release fence; nothing
// ever waits on another workgroup.
#pragma once
#include <algorithm>

#include "rows.hpp"

namespace moe {

// =================================================================== expert list
// Builds, in LDS, the set of selected experts in increasing id order and a token mask
// per expert. Entries outside [0, E) are ignored. Returns the number of experts.
__device__ __forceinline__ int build_list(const ExpertArgs& a, uint64_t* tmask, int* act, int* ids_l, int* scan) {
  const int P = a.T * a.k;
  for (int i = threadIdx.x; i < a.E; i += kBlock) tmask[i] = 0ull;
  for (int i = threadIdx.x; i < P; i += kBlock) ids_l[i] = a.ids[i];
  __syncthreads();
  for (int i = threadIdx.x; i < P; i += kBlock) {
    const int e = ids_l[i];
    if ((unsigned)e < (unsigned)a.E) atomicOr(reinterpret_cast<unsigned long long*>(&tmask[e]), 1ull << (i / a.k));
  }
  __syncthreads();
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int per = (a.E + kBlock - 1) / kBlock;
  const int b0 = threadIdx.x * per;
  int cnt = 0;
  for (int q = 0; q < per; ++q) cnt += (b0 + q < a.E && tmask[b0 + q] != 0ull) ? 1 : 0;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) scan[wave] = incl;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += scan[w];
  int r = base + incl - cnt;
  for (int q = 0; q < per; ++q)
    if (b0 + q < a.E && tmask[b0 + q] != 0ull) act[r++] = b0 + q;
  const int nact = scan[0] + scan[1] + scan[2] + scan[3];
  __syncthreads();
  return nact;
}

// Tokens of expert e (increasing) and their pair index t*k + j.
__device__ __forceinline__ int expert_tokens(const ExpertArgs& a, int e, const uint64_t* tmask, const int* ids_l,
                             int* tok, int* pair) {
  const uint64_t m = tmask[e];
  const int t = threadIdx.x;
  if (t < a.T && ((m >> t) & 1ull)) {
    const int pos = __popcll(m & ((1ull << t) - 1ull));
    int j = 0;
    while (j < a.k - 1 && ids_l[t * a.k + j] != e) ++j;
    tok[pos] = t;
    pair[pos] = t * a.k + j;
  }
  __syncthreads();
  return __popcll(m);
}

// ===================================================================== GEMV core
// Byte address of element `el` of a weight row.
template <int FMT>
__device__ __forceinline__ int64_t elem_byte(int el) {
  return FMT == W_BF16 ? 2 * (int64_t)el : (FMT == W_MXFP8 ? (int64_t)el : (int64_t)(el >> 1));
}

// LDS byte offset of the 16-byte sub-piece `sub` of piece `pc` (chunk-relative) for
// lane-in-row jl: consecutive lanes read consecutive 16-byte slots.
__device__ __forceinline__ int act_slot(int pc, int sub, int nsub, int LPR) {
  const int jl = pc % LPR, pass = pc / LPR;
  return ((pass * nsub + sub) * LPR + jl) * 16;
}

// Stage the activation chunk [kc0, kc0 + KC) of nt tokens into LDS.
//   AK = 0: BF16 values (exact), 8 per slot;  AK = 1: FP32 values, 4 per slot.
// src(t, el) returns the 16-byte slot content for token t and absolute element el.
template <int AK, int EPL, class Src>
__device__ __forceinline__ void stage_chunk(uint8_t* tile, const GemvMap& m, int kc0, int nt, Src src) {
  constexpr int PER = AK == 0 ? 8 : 4;
  constexpr int NSUB = EPL / PER;
  const int units = m.KC / PER;
  for (int u = threadIdx.x; u < nt * units; u += kBlock) {
    const int t = u / units, el = (u % units) * PER;
    const int pc = el / EPL, sub = (el % EPL) / PER;
    *reinterpret_cast<uint4*>(tile + t * m.KC * m.esize + act_slot(pc, sub, NSUB, m.LPR)) =
        src(t, kc0 + el);
  }
}

// acc[q][t] += row_q(piece) . act(t, piece) for one 16-byte weight piece per row.
template <int FMT, int AK, int NT, int RPL>
__device__ __forceinline__ void accumulate_piece(const uint4 (&wv)[RPL], const uint32_t (&sv)[RPL],
                                                 const uint8_t* tile, const GemvMap& m, int s,
                                                 int jl, float (&acc)[RPL][NT]) {
  constexpr int EPL = elems_per_piece(FMT);
  constexpr int NSUB = AK == 0 ? EPL / 8 : EPL / 4;
  const int tstride = m.KC * m.esize;
  const uint8_t* base = tile + ((s * NSUB) * m.LPR + jl) * 16;
  const int sstride = m.LPR * 16;  // next sub-piece of the same piece
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

// One workgroup computes R rows x nt tokens of  out = W[rows] . act  for expert e.
// row_of(r) maps a local row (0..R-1) to the weight row. Results (FP32, unscaled) go to
// sink(t, r, value) from the lane that owns the row.
template <int FMT, int AK, int NT, int RPL, class RowOf, class Stage, class Sink>
__device__ __forceinline__ void gemv_tile(const WTensor& W, const GemvMap& m, int e, uint8_t* tile,
                                          RowOf row_of, Stage stage, Sink sink) {
  constexpr int EPL = elems_per_piece(FMT);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int grp = lane / m.LPR, jl = lane % m.LPR;
  const uint8_t* rp[RPL];
  const uint8_t* sp[RPL];
  int rloc[RPL];
#pragma unroll
  for (int q = 0; q < RPL; ++q) {
    rloc[q] = (wave * m.G + grp) * RPL + q;
    const int64_t row = (int64_t)e * W.rows + row_of(rloc[q]);
    rp[q] = W.codes + row * W.code_row_bytes;
    sp[q] = W.scales ? W.scales + row * W.scale_row_bytes : nullptr;
  }
  float acc[RPL][NT];
#pragma unroll
  for (int q = 0; q < RPL; ++q)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[q][t] = 0.0f;

  for (int kc0 = 0; kc0 < W.K; kc0 += m.KC) {
    constexpr int NPMAX = RPL >= 4 ? 2 : 4;   // at most 8 weight pieces in flight per lane
    uint4 wv[NPMAX][RPL];
    uint32_t sv[NPMAX][RPL];
#pragma unroll
    for (int s = 0; s < NPMAX; ++s) {
      if (s < m.NP) {
        const int el = kc0 + (s * m.LPR + jl) * EPL;
#pragma unroll
        for (int q = 0; q < RPL; ++q) {
          wv[s][q] = load_stream16(rp[q] + elem_byte<FMT>(el));
          if constexpr (FMT == W_NVFP4)
            sv[s][q] = *reinterpret_cast<const uint16_t*>(sp[q] + (el >> 4));
          else if constexpr (FMT == W_MXFP4 || FMT == W_MXFP8)
            sv[s][q] = sp[q][el >> 5];
          else
            sv[s][q] = 0u;
        }
      }
    }
    stage(kc0);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NPMAX; ++s)
      if (s < m.NP) accumulate_piece<FMT, AK, NT, RPL>(wv[s], sv[s], tile, m, s, jl, acc);
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < RPL; ++q)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float v = acc[q][t];
      for (int o = m.LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
      if (jl == 0) sink(t, rloc[q], v);
    }
}

// Runs gemv_tile over all token groups of an item, dispatching the compile-time token
// count and rows-per-lane. group(tg, nt) sets up the group; done(tg, nt) is the epilogue.
template <int FMT, int AK, int MAXRPL, class RowOf, class StageF, class Sink, class Done>
__device__ __forceinline__ void gemv_item(const WTensor& W, const GemvMap& m, int e, uint8_t* tile,
                                          int n, RowOf row_of, StageF stage_for, Sink sink_for,
                                          Done done) {
  for (int tg = 0; tg < n; tg += m.NG) {
    const int nt = min(m.NG, n - tg);
    auto stage = [&](int kc0) { stage_for(kc0, tg, nt); };
    auto sink = [&](int t, int r, float v) { if (t < nt) sink_for(tg + t, r, v); };
#define MOE_RUN(NT_, RPL_) gemv_tile<FMT, AK, NT_, RPL_>(W, m, e, tile, row_of, stage, sink)
#define MOE_RUN_NT(RPL_)                    \
    if (nt == 1) MOE_RUN(1, RPL_);          \
    else if (nt == 2) MOE_RUN(2, RPL_);     \
    else MOE_RUN(4, RPL_);
    if (MAXRPL >= 4 && m.RPL == 4) { MOE_RUN_NT(4) }
    else if (MAXRPL >= 2 && m.RPL == 2) { MOE_RUN_NT(2) }
    else { MOE_RUN_NT(1) }
#undef MOE_RUN_NT
#undef MOE_RUN
    __syncthreads();
    done(tg, nt);
    __syncthreads();
  }
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

struct ExpertLds {
  uint64_t* tmask;
  int* act;
  int* ids;
  int* scan;   // [4] + flag at [4]
  int* tok;    // [64]
  int* pair;   // [64]
  float* tsc;  // [64]
  float* red;  // [4]
  uint8_t* tile;
  float* out;
};

__device__ __forceinline__ ExpertLds carve(const ExpertArgs& a, uint8_t* smem) {
  ExpertLds L;
  L.tmask = reinterpret_cast<uint64_t*>(smem);
  L.act = reinterpret_cast<int*>(L.tmask + a.E);
  L.ids = L.act + a.E;
  L.scan = L.ids + a.T * a.k;
  L.tok = L.scan + 8;
  L.pair = L.tok + 64;
  L.tsc = reinterpret_cast<float*>(L.pair + 64);
  L.red = L.tsc + 64;
  L.tile = smem + a.lds_list_bytes;
  L.out = reinterpret_cast<float*>(L.tile + a.lds_act_bytes);
  return L;
}

// ================================================================ gate/up kernel
template <int FMT>
__device__ __forceinline__ void gateup_item(const ExpertArgs& a, const ExpertLds& L, const WTensor& W,
                            const GemvMap& m, int e, int c, int n, int Iexp, bool routed) {
  const int RU = m.R / 2;
  const int i0 = c * RU;
  const float gsg = W.gscale ? W.gscale[(int64_t)e * W.gs_per_expert + 0] : 1.0f;
  const float gsu = W.gscale ? W.gscale[(int64_t)e * W.gs_per_expert + 1] : 1.0f;
  auto row_of = [&](int r) { return r < RU ? i0 + r : Iexp + i0 + r - RU; };
  const int afmt = routed ? a.afmt : A_BF16;
  auto stage_for = [&](int kc0, int tg, int nt) {
    const int* tok = L.tok + tg;
    if (afmt == A_NVFP4_4O6) {
      stage_chunk<0, elems_per_piece(FMT)>(L.tile, m, kc0, nt, [&](int t, int el) {
        const int tk = tok[t];
        return nvfp4_slot(a.xq_codes + (int64_t)tk * (a.H / 2), a.xq_scales + (int64_t)tk * (a.H / 16), el);
      });
    } else if (afmt == A_FP8_TOKEN) {
      stage_chunk<0, elems_per_piece(FMT)>(L.tile, m, kc0, nt, [&](int t, int el) {
        return fp8_slot(a.xq_codes + (int64_t)tok[t] * a.H, el);
      });
    } else {
      stage_chunk<0, elems_per_piece(FMT)>(L.tile, m, kc0, nt, [&](int t, int el) {
        return bf16_slot(a.x + (int64_t)tok[t] * a.H, el);
      });
    }
  };
  auto sink_for = [&](int t, int r, float v) { L.out[(t % m.NG) * m.R + r] = v; };
  auto done = [&](int tg, int nt) {
    for (int idx = threadIdx.x; idx < nt * RU; idx += kBlock) {
      const int tl = idx / RU, i = idx % RU, t = tg + tl;
      const float ts = L.tsc[t];
      const float gv = L.out[tl * m.R + i] * gsg * ts;
      const float uv = L.out[tl * m.R + RU + i] * gsu * ts;
      const float hv = gv / (1.0f + expf(-gv)) * uv;
      const int64_t off = (int64_t)L.pair[t] * a.hs + i0 + i;
      a.h[off] = hv;
      if (a.dbg_h) a.dbg_h[off] = hv;
    }
  };
  gemv_item<FMT, 0, 4>(W, m, e, L.tile, n, row_of, stage_for, sink_for, done);
}

// Re-quantize the h rows of one routed expert (all its pairs) per the layer's afmt.
__device__ __forceinline__ void quantize_expert_h(const ExpertArgs& a, const ExpertLds& L, int n) {
  for (int ti = 0; ti < n; ++ti) {
    const int p = L.pair[ti];
    const F32Row row{a.h + (int64_t)p * a.hs};
    if (a.afmt == A_NVFP4_4O6) {
      uint8_t* codes = a.hq_codes + (int64_t)p * (a.I / 2);
      uint8_t* scales = a.hq_scales + (int64_t)p * (a.I / 16);
      quant_row_nvfp4(row, a.I, codes, scales, a.hq_scale + p, nullptr, L.red);
      if (a.dbg_codes) quant_row_nvfp4(row, a.I, a.dbg_codes + (int64_t)p * (a.I / 2),
                                       a.dbg_scales + (int64_t)p * (a.I / 16), a.dbg_scale + p,
                                       nullptr, L.red);
    } else {
      quant_row_fp8(row, a.I, a.hq_codes + (int64_t)p * a.I, a.hq_scale + p, L.red);
      if (a.dbg_codes) quant_row_fp8(row, a.I, a.dbg_codes + (int64_t)p * a.I, a.dbg_scale + p, L.red);
    }
    __syncthreads();
  }
}

template <int RF, int SF>
__global__ void __launch_bounds__(kBlock, 2) gateup_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const ExpertLds L = carve(a, smem);
  const int routed_items = a.max_slots * a.rmap.nchunks;
  if ((int)blockIdx.x >= routed_items) {  // shared expert: independent of routing
    const int c = blockIdx.x - routed_items;
    for (int t = threadIdx.x; t < a.T; t += kBlock) {
      L.tok[t] = t;
      L.pair[t] = a.T * a.k + t;
      L.tsc[t] = 1.0f;
    }
    __syncthreads();
    gateup_item<SF>(a, L, a.sw, a.smap, 0, c, a.T, a.Ish, false);
    return;
  }
  const int u = blockIdx.x / a.rmap.nchunks, c = blockIdx.x % a.rmap.nchunks;
  const int nact = build_list(a, L.tmask, L.act, L.ids, L.scan);
  if (u >= nact) return;
  const int e = L.act[u];
  const int n = expert_tokens(a, e, L.tmask, L.ids, L.tok, L.pair);
  for (int t = threadIdx.x; t < n; t += kBlock)
    L.tsc[t] = a.afmt == A_BF16 ? 1.0f : a.xq_scale[L.tok[t]];
  __syncthreads();
  gateup_item<RF>(a, L, a.rw, a.rmap, e, c, n, a.I, true);
  if (a.afmt == A_BF16) return;
  // the last workgroup of this expert re-quantizes its h rows
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    L.scan[4] = atomicAdd(&a.counters[e], 1u) == (uint32_t)(a.rmap.nchunks - 1);
  __syncthreads();
  if (!L.scan[4]) return;
  __threadfence();
  quantize_expert_h(a, L, n);
  if (threadIdx.x == 0) a.counters[e] = 0u;
}

// =================================================================== down kernel
template <int FMT, int AK>
__device__ __forceinline__ void down_item(const ExpertArgs& a, const ExpertLds& L, const WTensor& W,
                          const GemvMap& m, int e, int c, int n, int Kexp, bool routed) {
  const int r0 = c * m.R;
  const float gs = W.gscale ? W.gscale[(int64_t)e * W.gs_per_expert] : 1.0f;
  auto row_of = [&](int r) { return r0 + r; };
  const int afmt = routed ? a.afmt : A_BF16;
  auto stage_for = [&](int kc0, int tg, int nt) {
    const int* pair = L.pair + tg;
    if constexpr (AK == 1) {
      stage_chunk<1, elems_per_piece(FMT)>(L.tile, m, kc0, nt, [&](int t, int el) {
        return f32_slot(a.h + (int64_t)pair[t] * a.hs, el);
      });
    } else {
      if (afmt == A_NVFP4_4O6) {
        stage_chunk<0, elems_per_piece(FMT)>(L.tile, m, kc0, nt, [&](int t, int el) {
          const int p = pair[t];
          return nvfp4_slot(a.hq_codes + (int64_t)p * (Kexp / 2), a.hq_scales + (int64_t)p * (Kexp / 16), el);
        });
      } else {
        stage_chunk<0, elems_per_piece(FMT)>(L.tile, m, kc0, nt, [&](int t, int el) {
          return fp8_slot(a.hq_codes + (int64_t)pair[t] * Kexp, el);
        });
      }
    }
  };
  auto sink_for = [&](int t, int r, float v) {
    a.o[(int64_t)L.pair[t] * a.H + r0 + r] = v * gs * L.tsc[t];
  };
  auto done = [](int, int) {};
  gemv_item<FMT, AK, 2>(W, m, e, L.tile, n, row_of, stage_for, sink_for, done);
}

template <int RF, int SF, int RAK>
__global__ void __launch_bounds__(kBlock, 2) down_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const ExpertLds L = carve(a, smem);
  const int nch = a.rmap.nchunks;  // equal for routed and shared (same R)
  const int routed_items = a.max_slots * nch;
  const int nact = build_list(a, L.tmask, L.act, L.ids, L.scan);
  int c;
  if ((int)blockIdx.x >= routed_items) {
    c = blockIdx.x - routed_items;
    for (int t = threadIdx.x; t < a.T; t += kBlock) {
      L.tok[t] = t;
      L.pair[t] = a.T * a.k + t;
      L.tsc[t] = 1.0f;
    }
    __syncthreads();
    down_item<SF, 1>(a, L, a.sw, a.smap, 0, c, a.T, a.Ish, false);
  } else {
    const int u = blockIdx.x / nch;
    c = blockIdx.x % nch;
    if (u >= nact) return;
    const int e = L.act[u];
    const int n = expert_tokens(a, e, L.tmask, L.ids, L.tok, L.pair);
    for (int t = threadIdx.x; t < n; t += kBlock)
      L.tsc[t] = a.afmt == A_BF16 ? 1.0f : a.hq_scale[L.pair[t]];
    __syncthreads();
    down_item<RF, RAK>(a, L, a.rw, a.rmap, e, c, n, a.I, true);
  }
  // the last workgroup of this hidden chunk combines every expert's output
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0)
    L.scan[4] = atomicAdd(&a.counters[c], 1u) == (uint32_t)(nact + a.has_shared - 1);
  __syncthreads();
  if (!L.scan[4]) return;
  __threadfence();
  const int R = a.rmap.R, r0 = c * R;
  for (int idx = threadIdx.x; idx < a.T * R; idx += kBlock) {
    const int t = idx / R, row = r0 + idx % R;
    float s = 0.0f;
    for (int j = 0; j < a.k; ++j) {
      const int p = t * a.k + j;
      s = fmaf(a.topk_w[p], __builtin_nontemporal_load(a.o + (int64_t)p * a.H + row), s);
    }
    if (a.has_shared) s += __builtin_nontemporal_load(a.o + (int64_t)(a.T * a.k + t) * a.H + row);
    a.y[(int64_t)t * a.H + row] = (uint16_t)f32_to_bf16_rne(s);
  }
  if (threadIdx.x == 0) a.counters[c] = 0u;
}

template <int RF, int SF>
hipError_t launch_experts_t(const ExpertArgs& gu, int gu_grid, size_t gu_lds,
                                   const ExpertArgs& dn, int dn_grid, size_t dn_lds, hipStream_t s) {
  hipLaunchKernelGGL((gateup_kernel<RF, SF>), dim3(gu_grid), dim3(kBlock), gu_lds, s, gu);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (dn.afmt == A_BF16)
    hipLaunchKernelGGL((down_kernel<RF, SF, 1>), dim3(dn_grid), dim3(kBlock), dn_lds, s, dn);
  else
    hipLaunchKernelGGL((down_kernel<RF, SF, 0>), dim3(dn_grid), dim3(kBlock), dn_lds, s, dn);
  return hipGetLastError();
}

}  // namespace moe
