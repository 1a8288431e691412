// Dequant-fused expert GEMVs for gfx950: gate/up with SwiGLU, down with the combine.
//
//   gateup_kernel  items = (shared expert, chunk of intermediate rows), then (selected
//                  expert, chunk); each lane holds a gate row and the matching up row,
//                  so SwiGLU is applied in registers; the last workgroup to finish a
//                  routed expert re-quantizes that expert's h rows when the layer
//                  quantizes h.
//   down_kernel    items = (shared or selected expert, chunk of hidden rows); the last
//                  workgroup to finish a hidden chunk combines every expert's partial
//                  output for it in a fixed order and writes BF16 y.
// Both kernels are persistent: a few resident workgroups per CU walk the item list
// (item = blockIdx.x, + gridDim.x, ...). An item stages the activations of its tokens
// (full K) in LDS once, then streams its weight rows in row-steps; the 16-byte weight
// pieces of the next step (possibly of the next item) are loaded while the current
// step computes. Weights are decoded in registers with the gfx950 FP4/FP8 converts.
// Hand-offs between workgroups use coherent stores/loads and a counter (device.hpp);
// nothing ever waits on another workgroup.
#pragma once
#include <algorithm>

#include "launch.hpp"
#include "rows.hpp"

namespace moe {

// =================================================================== expert list
// Builds, in LDS, the set of selected experts in increasing id order and a token mask
// per expert. Entries outside [0, E) are ignored. Returns the number of experts.
__device__ __forceinline__ int build_list(const ExpertArgs& a, uint64_t* tmask, int* act,
                                          int* ids_l, int* scan) {
  const int P = a.T * a.k;
  for (int i = threadIdx.x; i < a.E; i += kBlock) tmask[i] = 0ull;
  for (int i = threadIdx.x; i < P; i += kBlock) ids_l[i] = a.ids[i];
  __syncthreads();
  for (int i = threadIdx.x; i < P; i += kBlock) {
    const int e = ids_l[i];
    if ((unsigned)e < (unsigned)a.E)
      atomicOr(reinterpret_cast<unsigned long long*>(&tmask[e]), 1ull << (i / a.k));
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

// Tokens of expert e (increasing) and their pair index t*k + j, into LDS.
__device__ __forceinline__ int expert_tokens(const ExpertArgs& a, int e, const uint64_t* tmask,
                                             const int* ids_l, int* tok, int* pair) {
  const uint64_t m = tmask[e];
  const int t = threadIdx.x;
  if (t < a.T && ((m >> t) & 1ull)) {
    const int pos = __popcll(m & ((1ull << t) - 1ull));
    int j = 0;
    while (j < a.k - 1 && ids_l[t * a.k + j] != e) ++j;
    tok[pos] = t;
    pair[pos] = t * a.k + j;
  }
  return __popcll(m);
}

struct ExpertLds {
  uint64_t* tmask;
  int* act;
  int* ids;
  int* scan;   // [4] + a flag at [4]
  int* tok;    // [64]
  int* pair;   // [64]
  float* tsc;  // [64]
  float* red;  // [4]
  uint8_t* tile;
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

// Loads batch b (pieces b*NPB .. b*NPB + NPB - 1) of the lane's rows.
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
      if (i < m.NPB) {
        const int el = ((b * m.NPB + i) * m.LPR + jl) * EPL;
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
}

// Walks items first, first + gridDim.x, ... < n_items of one weight class. Call-backs
// (workgroup-uniform):
//   rows(item, step, lrow, out[RPL])  global weight rows (expert * rows + row) of this
//                                     lane's RPL rows at row-step `step`
//   setup(item) -> token count        fills the LDS token tables (synchronizes)
//   stage(item, tg, nt)               fills the LDS activation tile (no sync needed)
//   sink(item, tg, step, lrow, nt, acc)  results of the lanes with jl == 0
//   finish(item)                      item epilogue (hand-offs)
template <int FMT, int AK, int RPL, class Rows, class Setup, class Stage, class Sink, class Finish>
__device__ __forceinline__ void gemv_loop(const WTensor& W, const GemvMap& m, uint8_t* tile,
                                          int first, int n_items, Rows rows, Setup setup,
                                          Stage stage, Sink sink, Finish finish) {
  if (first >= n_items) return;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int grp = lane / m.LPR, jl = lane % m.LPR;
  const int lrow = wave * m.G + grp;   // row slot of this lane within a row-step
  const int tstride = W.K * m.esize;
  WeightRegs<RPL> cur;
  int64_t rr[RPL];
  int item = first;
  rows(item, 0, lrow, rr);
  fetch_batch<FMT, RPL>(W, m, rr, 0, jl, cur);
  while (true) {
    const int n = setup(item);
    for (int tg = 0; tg < n; tg += m.NG) {
      const int nt = min(m.NG, n - tg);
      stage(item, tg, nt);
      __syncthreads();
      for (int step = 0; step < m.NSTEP; ++step) {
        float acc[RPL][4];
#pragma unroll
        for (int q = 0; q < RPL; ++q)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[q][t] = 0.0f;
        for (int b = 0; b < m.NB; ++b) {
          // the next pipeline step: next batch, next row-step, next token group or next item
          int nitem = item, nstep = step, nb = b + 1;
          bool more = true;
          if (nb == m.NB) {
            nb = 0;
            if (++nstep == m.NSTEP) {
              nstep = 0;
              if (tg + m.NG >= n) {
                nitem = item + (int)gridDim.x;
                more = nitem < n_items;
              }
            }
          }
          WeightRegs<RPL> nxt;
          if (more) {
            int64_t nr[RPL];
            rows(nitem, nstep, lrow, nr);
            fetch_batch<FMT, RPL>(W, m, nr, nb, jl, nxt);
          }
#pragma unroll
          for (int i = 0; i < WeightRegs<RPL>::NPB; ++i) {
            if (i < m.NPB) {
              const int s = b * m.NPB + i;
              if (nt == 1) accumulate_piece<FMT, AK, 1, RPL>(cur.w[i], cur.s[i], tile, tstride, m.LPR, s, jl, acc);
              else if (AK == 1 || nt == 2) accumulate_piece<FMT, AK, 2, RPL>(cur.w[i], cur.s[i], tile, tstride, m.LPR, s, jl, acc);
              else accumulate_piece<FMT, AK, 4, RPL>(cur.w[i], cur.s[i], tile, tstride, m.LPR, s, jl, acc);
            }
          }
          if (more) cur = nxt;
        }
#pragma unroll
        for (int q = 0; q < RPL; ++q)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            if (t < nt) {
              float v = acc[q][t];
              for (int o = m.LPR / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
              acc[q][t] = v;
            }
          }
        if (jl == 0) sink(item, tg, step, lrow, nt, acc);
      }
      __syncthreads();   // the tile is restaged by the next group or item
    }
    finish(item);
    item += gridDim.x;
    if (item >= n_items) break;
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

// Items are numbered shared chunks first, then (routed expert, chunk); workgroup b takes
// items b, b + gridDim.x, ... of that numbering.
__device__ __forceinline__ int first_of_class(int class_base) {
  const int G = gridDim.x;
  return (((int)blockIdx.x - class_base) % G + G) % G;
}

// Token tables for the item's expert: routed experts from the list, the shared expert
// takes every token (pairs T*k + t).
__device__ __forceinline__ int setup_tokens(const ExpertArgs& a, const ExpertLds& L, bool routed,
                                            int e) {
  int n;
  if (routed) {
    n = expert_tokens(a, e, L.tmask, L.ids, L.tok, L.pair);
  } else {
    n = a.T;
    for (int t = threadIdx.x; t < n; t += kBlock) {
      L.tok[t] = t;
      L.pair[t] = a.T * a.k + t;
    }
  }
  __syncthreads();
  return n;
}

// ================================================================ gate/up kernel
// Re-quantize the h rows of one routed expert (all its pairs) per the layer's afmt.
// The rows were written by other workgroups of this launch (coherent loads).
__device__ __forceinline__ void quantize_expert_h(const ExpertArgs& a, const ExpertLds& L, int n) {
  for (int ti = 0; ti < n; ++ti) {
    const int p = L.pair[ti];
    const F32RowCoherent row{a.h + (int64_t)p * a.hs};
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

// Gate/up rows: lane row slot lrow at step `step` of chunk c is intermediate index
// i = c * RU + step * PS + lrow (PS = 4 * G pairs per step, RU = PS * NSTEP); the lane
// holds gate row i (q = 0) and up row I + i (q = 1).
template <int FMT>
__device__ __forceinline__ void gateup_class(const ExpertArgs& a, const ExpertLds& L, bool routed,
                                             int first, int n_items) {
  const WTensor& W = routed ? a.rw : a.sw;
  const GemvMap& m = routed ? a.rmap : a.smap;
  const int nch = m.nchunks, PS = 4 * m.G, RU = PS * m.NSTEP;
  const int Iexp = routed ? a.I : a.Ish;
  const int afmt = routed ? a.afmt : A_BF16;
  const bool coherent_h = routed && a.afmt != A_BF16;   // h is handed to the quantizer
  auto expert_of = [&](int item) { return routed ? L.act[item / nch] : 0; };
  auto rows = [&](int item, int step, int lrow, int64_t (&out)[2]) {
    const int64_t base = (int64_t)expert_of(item) * W.rows;
    const int i = (item % nch) * RU + step * PS + lrow;
    out[0] = base + i;
    out[1] = base + Iexp + i;
  };
  auto setup = [&](int item) {
    const int n = setup_tokens(a, L, routed, expert_of(item));
    for (int t = threadIdx.x; t < n; t += kBlock)
      L.tsc[t] = afmt == A_BF16 ? 1.0f : a.xq_scale[L.tok[t]];
    __syncthreads();
    return n;
  };
  auto stage = [&](int, int tg, int nt) {
    const int* tok = L.tok + tg;
    if (afmt == A_NVFP4_4O6) {
      stage_tile<0, elems_per_piece(FMT)>(L.tile, m, a.H, nt, [&](int t, int el) {
        const int tk = tok[t];
        return nvfp4_slot(a.xq_codes + (int64_t)tk * (a.H / 2), a.xq_scales + (int64_t)tk * (a.H / 16), el);
      });
    } else if (afmt == A_FP8_TOKEN) {
      stage_tile<0, elems_per_piece(FMT)>(L.tile, m, a.H, nt, [&](int t, int el) {
        return fp8_slot(a.xq_codes + (int64_t)tok[t] * a.H, el);
      });
    } else {
      stage_tile<0, elems_per_piece(FMT)>(L.tile, m, a.H, nt, [&](int t, int el) {
        return bf16_slot(a.x + (int64_t)tok[t] * a.H, el);
      });
    }
  };
  auto sink = [&](int item, int tg, int step, int lrow, int nt, const float (&acc)[2][4]) {
    const int e = expert_of(item);
    const int i = (item % nch) * RU + step * PS + lrow;
    const float gsg = W.gscale ? W.gscale[(int64_t)e * W.gs_per_expert + 0] : 1.0f;
    const float gsu = W.gscale ? W.gscale[(int64_t)e * W.gs_per_expert + 1] : 1.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nt) {
        const float ts = L.tsc[tg + t];
        const float gv = acc[0][t] * gsg * ts;
        const float uv = acc[1][t] * gsu * ts;
        const float hv = gv / (1.0f + expf(-gv)) * uv;
        const int64_t off = (int64_t)L.pair[tg + t] * a.hs + i;
        if (coherent_h) store_coherent(a.h + off, hv);
        else a.h[off] = hv;
        if (a.dbg_h) a.dbg_h[off] = hv;
      }
    }
  };
  auto finish = [&](int item) {
    if (!coherent_h) return;
    const int e = expert_of(item);
    if (arrive_last(&a.counters[e], (uint32_t)nch, &L.scan[4])) {
      const int n = setup_tokens(a, L, true, e);
      quantize_expert_h(a, L, n);
    }
  };
  gemv_loop<FMT, 0, 2>(W, m, L.tile, first, n_items, rows, setup, stage, sink, finish);
}

template <int RF, int SF>
__global__ void __launch_bounds__(kBlock, 2) gateup_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const ExpertLds L = carve(a, smem);
  const int nact = build_list(a, L.tmask, L.act, L.ids, L.scan);
  const int ns = a.has_shared ? a.smap.nchunks : 0;
  if (a.has_shared) gateup_class<SF>(a, L, false, blockIdx.x, ns);
  gateup_class<RF>(a, L, true, first_of_class(ns), nact * a.rmap.nchunks);
}

// =================================================================== down kernel
// Combine of one hidden chunk: y[t][row] = sum_j w[t][j] * o[t*k+j][row] + o_shared[t][row]
// in that order, FP32, rounded to BF16. The o rows come from every workgroup of this
// launch (coherent loads).
__device__ __forceinline__ void combine_chunk(const ExpertArgs& a, int c, int CH) {
  const int r0 = c * CH;
  for (int idx = threadIdx.x; idx < a.T * CH; idx += kBlock) {
    const int t = idx / CH, row = r0 + idx % CH;
    float s = 0.0f;
    for (int j = 0; j < a.k; ++j) {
      const int p = t * a.k + j;
      s = fmaf(a.topk_w[p], load_coherent(a.o + (int64_t)p * a.H + row), s);
    }
    if (a.has_shared) s += load_coherent(a.o + (int64_t)(a.T * a.k + t) * a.H + row);
    a.y[(int64_t)t * a.H + row] = (uint16_t)f32_to_bf16_rne(s);
  }
}

// Down rows: lane row slot lrow, row q, at step `step` of hidden chunk c is hidden row
// c * CH + step * RS + lrow * RPL + q (CH = RS * NSTEP, equal for routed and shared).
template <int FMT, int AK, int RPL>
__device__ __forceinline__ void down_loop(const ExpertArgs& a, const ExpertLds& L, bool routed,
                                          int nact, int first, int n_items) {
  const WTensor& W = routed ? a.rw : a.sw;
  const GemvMap& m = routed ? a.rmap : a.smap;
  const int nch = m.nchunks, RS = m.RS, CH = RS * m.NSTEP;
  const int Kexp = routed ? a.I : a.Ish;
  const int afmt = routed ? a.afmt : A_BF16;
  auto expert_of = [&](int item) { return routed ? L.act[item / nch] : 0; };
  auto rows = [&](int item, int step, int lrow, int64_t (&out)[RPL]) {
    const int64_t base = (int64_t)expert_of(item) * W.rows + (item % nch) * CH + step * RS + lrow * RPL;
#pragma unroll
    for (int q = 0; q < RPL; ++q) out[q] = base + q;
  };
  auto setup = [&](int item) {
    const int n = setup_tokens(a, L, routed, expert_of(item));
    for (int t = threadIdx.x; t < n; t += kBlock)
      L.tsc[t] = afmt == A_BF16 ? 1.0f : a.hq_scale[L.pair[t]];
    __syncthreads();
    return n;
  };
  auto stage = [&](int, int tg, int nt) {
    const int* pair = L.pair + tg;
    if constexpr (AK == 1) {
      stage_tile<1, elems_per_piece(FMT)>(L.tile, m, Kexp, nt, [&](int t, int el) {
        return f32_slot(a.h + (int64_t)pair[t] * a.hs, el);
      });
    } else {
      if (afmt == A_NVFP4_4O6) {
        stage_tile<0, elems_per_piece(FMT)>(L.tile, m, Kexp, nt, [&](int t, int el) {
          const int p = pair[t];
          return nvfp4_slot(a.hq_codes + (int64_t)p * (Kexp / 2), a.hq_scales + (int64_t)p * (Kexp / 16), el);
        });
      } else {
        stage_tile<0, elems_per_piece(FMT)>(L.tile, m, Kexp, nt, [&](int t, int el) {
          return fp8_slot(a.hq_codes + (int64_t)pair[t] * Kexp, el);
        });
      }
    }
  };
  auto sink = [&](int item, int tg, int step, int lrow, int nt, const float (&acc)[RPL][4]) {
    const int e = expert_of(item);
    const float gs = W.gscale ? W.gscale[(int64_t)e * W.gs_per_expert] : 1.0f;
    const int row0 = (item % nch) * CH + step * RS + lrow * RPL;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nt) {
        const float sc = gs * L.tsc[tg + t];
        float* o = a.o + (int64_t)L.pair[tg + t] * a.H + row0;
#pragma unroll
        for (int q = 0; q < RPL; ++q) store_coherent(o + q, acc[q][t] * sc);
      }
    }
  };
  auto finish = [&](int item) {
    const int c = item % nch;
    if (arrive_last(&a.counters[c], (uint32_t)(nact + a.has_shared), &L.scan[4])) combine_chunk(a, c, CH);
  };
  gemv_loop<FMT, AK, RPL>(W, m, L.tile, first, n_items, rows, setup, stage, sink, finish);
}

template <int FMT, int AK>
__device__ __forceinline__ void down_class(const ExpertArgs& a, const ExpertLds& L, bool routed,
                                           int nact, int first, int n_items) {
  const int rpl = routed ? a.rmap.RPL : a.smap.RPL;
  if (rpl == 2) down_loop<FMT, AK, 2>(a, L, routed, nact, first, n_items);
  else down_loop<FMT, AK, 1>(a, L, routed, nact, first, n_items);
}

template <int RF, int SF, int RAK>
__global__ void __launch_bounds__(kBlock, 2) down_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  const ExpertLds L = carve(a, smem);
  const int nact = build_list(a, L.tmask, L.act, L.ids, L.scan);
  const int nch = a.rmap.nchunks;  // equal for routed and shared (same chunk rows)
  const int ns = a.has_shared ? nch : 0;
  if (a.has_shared) down_class<SF, 1>(a, L, false, nact, blockIdx.x, ns);
  down_class<RF, RAK>(a, L, true, nact, first_of_class(ns), nact * nch);
}

// ================================================================ host launchers
template <int RF, int SF>
hipError_t launch_experts_t(const ExpertArgs& gu, int gu_grid, size_t gu_lds,
                            const ExpertArgs& dn, int dn_grid, size_t dn_lds, hipStream_t s) {
  hipError_t err = launch_kernel(K_GATEUP, gateup_kernel<RF, SF>, dim3(gu_grid), dim3(kBlock), gu_lds, s, gu);
  if (err != hipSuccess) return err;
  if (dn.afmt == A_BF16)
    return launch_kernel(K_DOWN, down_kernel<RF, SF, 1>, dim3(dn_grid), dim3(kBlock), dn_lds, s, dn);
  return launch_kernel(K_DOWN, down_kernel<RF, SF, 0>, dim3(dn_grid), dim3(kBlock), dn_lds, s, dn);
}

}  // namespace moe
