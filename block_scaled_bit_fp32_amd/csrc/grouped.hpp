// Grouped expert kernels for batches of 32 tokens and more (gfx950 MFMA).
//
// The same work split as the GEMV kernels (experts.hpp: shared-expert workgroups,
// per-workgroup cost spans over the units of the selected experts), with units of up
// to 32 tokens, so an expert's weights are read once per 32 of its tokens instead of
// once per 4. Each wave owns 32 weight rows of a row tile and computes them against
// the unit's (up to) 32 tokens with v_mfma_f32_32x32x16_bf16:
//   A (32 rows x 16 K): weights, decoded exactly to BF16 in registers (E2M1 and E4M3
//     values times their block scale have at most 6 significant bits);
//   B (16 K x 32 tokens): activations, staged per K stage in LDS as BF16 (BF16 tokens,
//     decoded NVFP4 / FP8 activations, and h, which the gate/up kernel stores as BF16
//     where it is not re-quantized, as the GEMV kernels do);
//   accumulation in FP32. Lane l holds row l % 32 of A and token l % 32 of B and takes
//   its K elements from half l / 32 of the stage; A and B use the same K order, which
//   is all the dot products need.
// Weights: a stage is 128 bytes of each of the workgroup's 128 rows. They are loaded
// coalesced (each load covers 8 rows x 128 contiguous bytes), one stage ahead in
// registers, and written to an LDS tile after the current stage's MFMAs; each lane then
// reads its 64 bytes in the MFMA layout from there. Loading the MFMA layout directly
// (a lane reads 64 bytes of one row, a wave 32 rows) reads far slower on this chip. The
// next stage's activations and scales are loaded before those weights and stored to the
// other LDS buffer after the current stage's MFMAs.
#pragma once
#include "experts.hpp"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

constexpr int kGTok = 32;        // tokens per unit (MFMA N)
constexpr int kGActSlots = 8;    // 16-byte activation slots per thread per stage

// One stage's raw operands of this lane: weights, their block scales, and the
// activation slots this thread stages for the workgroup.
struct GStage {
  uint4 w[4];
  uint2 sc;
  uint4 act[kGActSlots];
  float tsc;                     // the scale of this lane's token (stage 0 of a tile)
  float gs[2];                   // the expert's global weight scales (stage 0)
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(v.x, v.y, v.z, v.w));
}
__device__ __forceinline__ bf16x8_t pack_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8_t, make_uint4(a, b, c, d));
}
// Upper 16 bits of two FP32 values as a BF16 pair (exact when the values fit BF16).
__device__ __forceinline__ uint32_t trunc_pair(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// A fragment of MFMA step s: the lane's weight elements [8s, 8s + 8) of the stage, as BF16.
template <int FMT>
__device__ __forceinline__ bf16x8_t weight_frag(const GStage& g, int s) {
  if constexpr (FMT == W_BF16) {
    return as_bf16x8(g.w[s]);
  } else if constexpr (FMT == W_MXFP8) {
    // 8 E4M3 bytes [8s, 8s + 8); E8M0 scale per 32 elements
    const uint4 q = g.w[s >> 1];
    const uint32_t lo = (s & 1) ? q.z : q.x, hi = (s & 1) ? q.w : q.y;
    const float sc = e8m0_to_f32((g.sc.x >> (8 * (s >> 2))) & 0xFFu);
    return pack_bf16x8(as_u32(fp8x2_to_bf16<false>(lo, sc)), as_u32(fp8x2_to_bf16<true>(lo, sc)),
                       as_u32(fp8x2_to_bf16<false>(hi, sc)), as_u32(fp8x2_to_bf16<true>(hi, sc)));
  } else {
    // 8 E2M1 nibbles = bytes [4s, 4s + 4)
    const uint4 q = g.w[s >> 2];
    const uint32_t word = (s & 3) == 0 ? q.x : (s & 3) == 1 ? q.y : (s & 3) == 2 ? q.z : q.w;
    if constexpr (FMT == W_MXFP4) {
      const float sc = e8m0_to_f32((g.sc.x >> (8 * (s >> 2))) & 0xFFu);
      return pack_bf16x8(as_u32(fp4x2_to_bf16<0>(word, sc)), as_u32(fp4x2_to_bf16<1>(word, sc)),
                         as_u32(fp4x2_to_bf16<2>(word, sc)), as_u32(fp4x2_to_bf16<3>(word, sc)));
    } else {   // NVFP4: E4M3 scale per 16 elements, applied in FP32 (exact), then truncated
      const uint32_t sb = (s >> 1) < 4 ? (g.sc.x >> (8 * (s >> 1))) : (g.sc.y >> (8 * ((s >> 1) - 4)));
      const float S = e4m3_to_f32(sb & 0xFFu);
      const f32x2_t v0 = fp4x2_to_f32<0>(word, 1.0f), v1 = fp4x2_to_f32<1>(word, 1.0f);
      const f32x2_t v2 = fp4x2_to_f32<2>(word, 1.0f), v3 = fp4x2_to_f32<3>(word, 1.0f);
      return pack_bf16x8(trunc_pair(v0.x * S, v0.y * S), trunc_pair(v1.x * S, v1.y * S),
                         trunc_pair(v2.x * S, v2.y * S), trunc_pair(v3.x * S, v3.y * S));
    }
  }
}

// Walks one workgroup's span of a class. `row_of(e, tile, r)` is the weight row of
// this wave's row r (0..31) of row tile `tile` of expert e; `op` is the class's
// GateupOps / DownOps (activation loads and scales); `sink(cx, tile, acc, tsc, gs)`
// consumes a finished row tile (lane token l % 32, rows per the MFMA layout).
template <int FMT, class Ops, class RowOf, class Sink>
__device__ __forceinline__ void walk_grouped(const WTensor& W, const GroupMap& gm, const ExpertLds& L,
                                             const ClassTab& C, const Span& sp, const Ops& op, RowOf row_of,
                                             Sink sink) {
  constexpr int PER = 8;                  // staged BF16 elements per 16-byte slot
  constexpr int KS = group_ks(FMT);
  constexpr int SPR = KS / PER;           // slots per staged token row
  constexpr int NSTEP = KS / 16;          // MFMA steps per stage
  static_assert(kGTok * SPR <= kGActSlots * kBlock, "stage does not fit the staging slots");
  if (sp.left <= 0) return;
  int left = sp.left;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int half = lane >> 5, lr = lane & 31;
  const ClassCost k{gm.NG, gm.steps, gm.cw, gm.ct};
  auto advance = [&](Cursor& p) {
    if (++p.b < gm.NS) return;
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
  // loads of one position: activation slots and (stage 0) scales first, weights last
  auto fetch = [&](const Cursor& p, GStage& g) {
    const int crow = p.rb + p.g * k.NG, n = min(k.NG, p.n - p.g * k.NG);
#pragma unroll
    for (int i = 0; i < kGActSlots; ++i) {
      const int u = i * kBlock + threadIdx.x;
      const int j = u / SPR, c = u % SPR;
      g.act[i] = make_uint4(0u, 0u, 0u, 0u);
      if (u < kGTok * SPR && j < n)
        g.act[i] = op.ld(C.r_tok[crow + j], C.r_pair[crow + j], p.b * KS + c * PER);
    }
    if (p.b == 0) {
      g.tsc = lr < n ? op.tsc(C.r_tok[crow + lr], C.r_pair[crow + lr]) : 0.0f;
      g.gs[0] = op.gs(p.e, 0);
      g.gs[1] = op.gs(p.e, 1);
    }
    // weights: load q covers rows 8q .. 8q + 7 of the wave's 32, 128 contiguous bytes each
    // (the stage's part of the row); lane l takes 16-byte chunk (l % 8) ^ (row % 8) of row
    // 8q + l / 8, which is where it lands in the LDS tile (see store)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 8 * q + (lane >> 3);
      const int64_t wr = row_of(p.e, p.s, r);
      g.w[q] = load_stream16(W.codes + wr * W.code_row_bytes + elem_byte<FMT>(p.b * KS) + 16 * ((lane ^ r) & 7));
    }
    const int64_t row = row_of(p.e, p.s, lr);
    const int k0 = p.b * KS + half * (KS / 2);
    if constexpr (FMT == W_NVFP4) {
      g.sc = *reinterpret_cast<const uint2*>(W.scales + row * W.scale_row_bytes + (k0 >> 4));
    } else if constexpr (FMT == W_MXFP4) {
      g.sc = make_uint2(*reinterpret_cast<const uint32_t*>(W.scales + row * W.scale_row_bytes + (k0 >> 5)), 0u);
    } else if constexpr (FMT == W_MXFP8) {
      g.sc = make_uint2(*reinterpret_cast<const uint16_t*>(W.scales + row * W.scale_row_bytes + (k0 >> 5)), 0u);
    } else {
      g.sc = make_uint2(0u, 0u);
    }
  };
  // stores of one position's staged data into LDS buffer `buf`
  float* s_tsc = L.w_tsc;       // [32] token scales of the current row tile
  float* s_gs = L.w_gs;         // [2] its expert's global scales
  // weight tile: [wave][32 rows][128 bytes], 16-byte chunk c of row r at slot c ^ (r % 8),
  // so that the 8 lanes of a read phase hit 8 different bank groups
  uint8_t* wlds = L.tile + 2 * (kGTok * gm.tstride);
  auto store = [&](const Cursor& p, const GStage& g, int buf) {
    uint8_t* wt = wlds + wave * (kGWeightStage / 4);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(wt + (8 * q + (lane >> 3)) * 128 + 16 * (lane & 7)) = g.w[q];
    uint8_t* tile = L.tile + buf * (kGTok * gm.tstride);
#pragma unroll
    for (int i = 0; i < kGActSlots; ++i) {
      const int u = i * kBlock + threadIdx.x;
      if (u < kGTok * SPR)
        *reinterpret_cast<uint4*>(tile + (u / SPR) * gm.tstride + (u % SPR) * 16) = op.cv(g.act[i]);
    }
    if (p.b == 0) {
      if (wave == 0 && half == 0) s_tsc[lr] = g.tsc;
      if (threadIdx.x == 0) { s_gs[0] = g.gs[0]; s_gs[1] = g.gs[1]; }
    }
  };
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  int buf = 0;
  auto do_step = [&](auto pf, const Cursor& p, GStage& cur, GStage& nxt, Cursor& np) {
    if constexpr (decltype(pf)::value) {
      np = p;
      advance(np);
      fetch(np, nxt);
    }
    const uint8_t* tile = L.tile + buf * (kGTok * gm.tstride) + lr * gm.tstride;
    GStage wc;   // this lane's 64 bytes of the stage (chunks 4 half .. 4 half + 3 of row lr)
    {
      const uint8_t* wt = wlds + wave * (kGWeightStage / 4) + lr * 128;
#pragma unroll
      for (int j = 0; j < 4; ++j) wc.w[j] = *reinterpret_cast<const uint4*>(wt + 16 * ((4 * half + j) ^ (lr & 7)));
      wc.sc = cur.sc;
    }
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      const bf16x8_t a = weight_frag<FMT>(wc, s);
      const int kk = half * (KS / 2) + 8 * s;   // K offset of this lane's B fragment
      const bf16x8_t b = as_bf16x8(*reinterpret_cast<const uint4*>(tile + kk * 2));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
    if (p.b == gm.NS - 1) {   // row tile done
      const int crow = p.rb + p.g * k.NG, n = min(k.NG, p.n - p.g * k.NG);
      sink(UnitCtx{crow, 0, n}, p.s, acc, s_tsc[lr], s_gs[0], s_gs[1]);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    }
    if constexpr (decltype(pf)::value) {
      if (np.b == 0) lds_barrier();   // every wave has read this tile's scales
      store(np, nxt, buf ^ 1);
    }
    lds_barrier();
    buf ^= 1;
  };
  Cursor pa{sp.a0, sp.g0, sp.s0, 0, sp.e0, sp.n0, sp.rb0}, pb = pa;
  GStage A, B;
  fetch(pa, A);
  store(pa, A, 0);
  lds_barrier();
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

// ------------------------------------------------ MX weights on the scaled MFMA
// MX weights (MXFP4, MXFP8) with 8- or 4-bit activations (FP8 per token, MXFP4, MXFP8)
// run on gfx950's v_mfma_scale_f32_32x32x64_f8f6f4: the E2M1 / E4M3 codes go in raw and
// each operand's E8M0 block scales ride in the instruction, so neither side is decoded.
// Operand layout of that instruction (checked on the GPU against a host reference for
// every pairing of FP8 and FP4 operands): lane l holds row (A) or column (B) l % 32 and
// half h = l / 32 of each 32-element K block: a 4-bit operand holds K [32 h, 32 h + 32)
// of the instruction's 64, an 8-bit operand holds K [16 h, 16 h + 16) in bytes 0..15 and
// K [32 + 16 h, 48 + 16 h) in bytes 16..31; the E8M0 scale of K block kb of row r comes
// from lane r + 32 kb. The walk maps each instruction's two K blocks onto two OCP scale
// blocks of the stage, the same on both operands:
//   MXFP4 weights (stage 256): instruction j, K block kb = stage elements 128 kb + 32 j;
//   MXFP8 weights (stage 128): instruction j, K block kb = stage elements 64 j + 32 kb.
// FP8-per-token activations take the unit scale (E8M0 127); their FP32 scale is applied
// in the epilogue. FP4 products are exact; the FP8 x FP8 instruction accumulates with
// about 1e-5 of the sum of |terms| of internal rounding (measured), far inside the
// layer's output tolerance.
template <int FMT, int AF>
constexpr bool use_scaled_mfma() {
  return (FMT == W_MXFP4 || FMT == W_MXFP8) && (AF == A_FP8_TOKEN || AF == A_MXFP4 || AF == A_MXFP8);
}
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// One v_mfma_scale_f32_32x32x64_f8f6f4 (operand formats FA, FB: 4 = E2M1 in 4 registers,
// 0 = E4M3 in 8). It is issued from inline assembly with its sources as the statement's
// inputs and 21 wait states after it inside the statement: the compiler's own scheduling
// of this instruction let later VALU writes land in its A, B and scale registers while
// the instruction was still reading them (seen in the generated code; a quarter of the
// outputs came out wrong), so here nothing may reuse the sources, or read the result,
// until the instruction is done with them.
template <int FA, int FB>
struct MfmaOperands {
  using A = typename std::conditional<FA == 4, i32x4_t, i32x8_t>::type;
  using B = typename std::conditional<FB == 4, i32x4_t, i32x8_t>::type;
};
template <int FA, int FB>
__device__ __forceinline__ void mfma_scale_32x32x64(f32x16_t& acc, const typename MfmaOperands<FA, FB>::A& a,
                                                    const typename MfmaOperands<FA, FB>::B& b, int sa, int sb) {
  asm volatile(
      "v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0] cbsz:%5 blgp:%6\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 4"
      : "+v"(acc)
      : "v"(a), "v"(b), "v"(sa), "v"(sb), "n"(FA), "n"(FB));
}

struct GStageMx {
  uint4 w[4];                    // 64 bytes of weight codes
  uint32_t sc;                   // their 4 E8M0 scale bytes
  uint4 act[2];                  // staged activation code slots of this thread
  uint2 asc;                     // a token's activation scale bytes of the stage (MX)
  float tsc;
  float gs[2];
};

template <int FMT, int AF, class Ops, class RowOf, class Sink>
__device__ __forceinline__ void walk_grouped_mx(const WTensor& W, const GroupMap& gm, const ExpertLds& L,
                                                const ClassTab& C, const Span& sp, const Ops& op, RowOf row_of,
                                                Sink sink) {
  constexpr int KS = group_ks(FMT);                 // 256 (FP4 weights) or 128 (FP8 weights)
  constexpr bool W4 = FMT == W_MXFP4;
  constexpr bool A4 = AF == A_MXFP4;
  constexpr bool AMX = AF == A_MXFP4 || AF == A_MXFP8;
  constexpr int ABYTES = A4 ? KS / 2 : KS;          // activation code bytes per token and stage
  constexpr int SPR = ABYTES / 16;                  // 16-byte slots per token and stage
  constexpr int NSLOT = (kGTok * SPR + kBlock - 1) / kBlock;
  constexpr int NI = KS / 64;                       // instructions per stage
  constexpr int SCB = KS / 32;                      // scale blocks per token and stage
  constexpr int FA = W4 ? 4 : 0, FB = A4 ? 4 : 0;   // operand formats: E2M1 4, E4M3 0
  static_assert(NSLOT <= 2, "activation slots");
  if (sp.left <= 0) return;
  int left = sp.left;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int half = lane >> 5, lr = lane & 31;
  const int tstride = gm.tstride;                   // ABYTES + 16
  const int bufbytes = kGTok * tstride + kGTok * 8;
  const ClassCost k{gm.NG, gm.steps, gm.cw, gm.ct};
  auto advance = [&](Cursor& p) {
    if (++p.b < gm.NS) return;
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
  auto fetch = [&](const Cursor& p, GStageMx& g) {
    const int crow = p.rb + p.g * k.NG, n = min(k.NG, p.n - p.g * k.NG);
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) {
      const int u = i * kBlock + threadIdx.x;
      const int j = u / SPR, c = u % SPR;
      g.act[i] = make_uint4(0u, 0u, 0u, 0u);
      if (u < kGTok * SPR && j < n)
        g.act[i] = ld16(op.codes_row(C.r_tok[crow + j], C.r_pair[crow + j]) + p.b * ABYTES + c * 16);
    }
    g.asc = make_uint2(0u, 0u);
    if constexpr (AMX) {
      if ((int)threadIdx.x < n) {
        const uint8_t* sr = op.scales_row(C.r_tok[crow + threadIdx.x], C.r_pair[crow + threadIdx.x]) + p.b * SCB;
        g.asc = SCB == 8 ? *reinterpret_cast<const uint2*>(sr) : make_uint2(*reinterpret_cast<const uint32_t*>(sr), 0u);
      }
    }
    if (p.b == 0) {
      g.tsc = lr < n ? op.tsc(C.r_tok[crow + lr], C.r_pair[crow + lr]) : 0.0f;
      g.gs[0] = op.gs(p.e, 0);
      g.gs[1] = op.gs(p.e, 1);
    }
    // weights coalesced as in walk_grouped: 128 bytes of the stage per row, through LDS
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 8 * q + (lane >> 3);
      const int64_t wr = row_of(p.e, p.s, r);
      g.w[q] = load_stream16(W.codes + wr * W.code_row_bytes + (W4 ? p.b * KS / 2 : p.b * KS) + 16 * ((lane ^ r) & 7));
    }
    const int64_t row = row_of(p.e, p.s, lr);
    const uint8_t* sp_ = W.scales + row * W.scale_row_bytes;
    if constexpr (W4) {   // this lane's elements [128 h, 128 h + 128) of the stage
      g.sc = *reinterpret_cast<const uint32_t*>(sp_ + ((p.b * KS + half * (KS / 2)) >> 5));
    } else {              // its bytes 16 h + 32 q of the stage (q < 4): both halves of each block
      g.sc = *reinterpret_cast<const uint32_t*>(sp_ + ((p.b * KS) >> 5));
    }
  };
  float* s_tsc = L.w_tsc;
  float* s_gs = L.w_gs;
  uint8_t* wlds = L.tile + 2 * bufbytes;   // weight tiles, laid out as in walk_grouped
  auto store = [&](const Cursor& p, const GStageMx& g, int buf) {
    uint8_t* wt = wlds + wave * (kGWeightStage / 4);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(wt + (8 * q + (lane >> 3)) * 128 + 16 * (lane & 7)) = g.w[q];
    uint8_t* tile = L.tile + buf * bufbytes;
#pragma unroll
    for (int i = 0; i < NSLOT; ++i) {
      const int u = i * kBlock + threadIdx.x;
      if (u < kGTok * SPR) *reinterpret_cast<uint4*>(tile + (u / SPR) * tstride + (u % SPR) * 16) = g.act[i];
    }
    if constexpr (AMX) {
      if ((int)threadIdx.x < kGTok) *reinterpret_cast<uint2*>(tile + kGTok * tstride + threadIdx.x * 8) = g.asc;
    }
    if (p.b == 0) {
      if (wave == 0 && half == 0) s_tsc[lr] = g.tsc;
      if (threadIdx.x == 0) { s_gs[0] = g.gs[0]; s_gs[1] = g.gs[1]; }
    }
  };
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
  int buf = 0;
  auto do_step = [&](auto pf, const Cursor& p, GStageMx& cur, GStageMx& nxt, Cursor& np) {
    if constexpr (decltype(pf)::value) {
      np = p;
      advance(np);
      fetch(np, nxt);
    }
    const uint8_t* tile = L.tile + buf * bufbytes;
    const uint8_t* arow = tile + lr * tstride;
    uint2 as2 = make_uint2(0u, 0u);
    if constexpr (AMX) as2 = *reinterpret_cast<const uint2*>(tile + kGTok * tstride + lr * 8);
    GStageMx wc;   // this lane's 64 bytes: chunks 4 h + j (FP4) or 2 j + h (FP8) of row lr
    {
      const uint8_t* wt = wlds + wave * (kGWeightStage / 4) + lr * 128;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = W4 ? 4 * half + j : 2 * j + half;
        wc.w[j] = *reinterpret_cast<const uint4*>(wt + 16 * (c ^ (lr & 7)));
      }
      wc.sc = cur.sc;
    }
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      typename MfmaOperands<FA, FB>::A a;
      int sa, blk;   // this lane's weight scale; the stage scale block it supplies
      if constexpr (W4) {
        a = i32x4_t{(int)wc.w[j].x, (int)wc.w[j].y, (int)wc.w[j].z, (int)wc.w[j].w};
        sa = (int)((wc.sc >> (8 * j)) & 0xFFu);
        blk = 4 * half + j;
      } else {
        a = i32x8_t{(int)wc.w[2 * j].x, (int)wc.w[2 * j].y, (int)wc.w[2 * j].z, (int)wc.w[2 * j].w,
                    (int)wc.w[2 * j + 1].x, (int)wc.w[2 * j + 1].y, (int)wc.w[2 * j + 1].z, (int)wc.w[2 * j + 1].w};
        blk = 2 * j + half;
        sa = (int)((wc.sc >> (8 * blk)) & 0xFFu);
      }
      typename MfmaOperands<FA, FB>::B b;
      if constexpr (A4) {   // 32 E2M1 of stage elements 32 blk.. (16 bytes)
        const uint4 v = *reinterpret_cast<const uint4*>(arow + 16 * blk);
        b = i32x4_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
      } else {              // E4M3: bytes 0..15 from K block 0's half, 16..31 from block 1's
        const int o0 = W4 ? 32 * j + 16 * half : 64 * j + 16 * half;
        const int o1 = W4 ? 128 + 32 * j + 16 * half : 64 * j + 32 + 16 * half;
        const uint4 v0 = *reinterpret_cast<const uint4*>(arow + o0);
        const uint4 v1 = *reinterpret_cast<const uint4*>(arow + o1);
        b = i32x8_t{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w, (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
      }
      int sb = 127;
      if constexpr (AMX) sb = (int)(((blk < 4 ? as2.x : as2.y) >> (8 * (blk & 3))) & 0xFFu);
      mfma_scale_32x32x64<FA, FB>(acc, a, b, sa, sb);
    }
    if (p.b == gm.NS - 1) {   // row tile done
      const int crow = p.rb + p.g * k.NG, n = min(k.NG, p.n - p.g * k.NG);
      sink(UnitCtx{crow, 0, n}, p.s, acc, s_tsc[lr], s_gs[0], s_gs[1]);
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    }
    if constexpr (decltype(pf)::value) {
      if (np.b == 0) lds_barrier();   // every wave has read this tile's scales
      store(np, nxt, buf ^ 1);
    }
    lds_barrier();
    buf ^= 1;
  };
  Cursor pa{sp.a0, sp.g0, sp.s0, 0, sp.e0, sp.n0, sp.rb0}, pb = pa;
  GStageMx A, B;
  fetch(pa, A);
  store(pa, A, 0);
  lds_barrier();
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

// Output row (0..31) of accumulator register r on this lane (32x32 MFMA layout).
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// ============================================================ grouped gate/up kernel
// Row tile t of an expert: intermediate indices [64 t, 64 t + 64), 16 per wave; a wave's
// rows 0..15 are gate rows, 16..31 the matching up rows, so accumulator registers r and
// r + 8 of a lane hold the gate and up value of the same (index, token).
template <int FMT, int AF>
__device__ __forceinline__ void ggateup_walk(const ExpertArgs& a, const ExpertLds& L, const ClassTab& C,
                                             bool routed, const Span& sp) {
  const WTensor& W = routed ? a.rw : a.sw;
  const GemvMap& m = routed ? a.rmap : a.smap;
  const GroupMap& gm = routed ? a.rgm : a.sgm;
  const int Iexp = routed ? a.I : a.Ish;
  const GateupOps<AF> op{a.x, a.xq_codes, a.xq_scales, a.xq_scale, W.gscale, W.gs_per_expert, W.rows, Iexp,
                         4 * m.G, a.H, a.hs, a.h, a.dbg_h, L.w_tsc, C.r_pair};
  const int wave = threadIdx.x / kWave, half = (threadIdx.x & (kWave - 1)) >> 5, lr = threadIdx.x & 31;
  auto row_of = [&](int e, int t, int r) -> int64_t {
    const int i = 64 * t + 16 * wave + (r & 15);
    return (int64_t)e * W.rows + (r < 16 ? i : Iexp + i);
  };
  auto sink = [&](const UnitCtx& cx, int t, const f32x16_t& acc, float ts, float gsg, float gsu) {
    if (lr >= cx.n) return;
    const int64_t off = (int64_t)C.r_pair[cx.crow + lr] * a.hs + 64 * t + 16 * wave;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const float gv = acc[r] * gsg * ts, uv = acc[r + 8] * gsu * ts;
      const float hv = gv / (1.0f + expf(-gv)) * uv;
      // an h that is not re-quantized is stored as BF16 at the byte position of its FP32
      // row, as the GEMV kernels store it (16-bit-activation layers, every shared expert)
      if constexpr (AF == A_BF16)
        reinterpret_cast<uint16_t*>(a.h)[off + (int64_t)C.r_pair[cx.crow + lr] * a.hs + acc_row(r, half)] =
            (uint16_t)f32_to_bf16_rne(hv);
      else
        a.h[off + acc_row(r, half)] = hv;
      if (a.dbg_h) a.dbg_h[off + acc_row(r, half)] = hv;
    }
  };
  if constexpr (use_scaled_mfma<FMT, AF>())
    walk_grouped_mx<FMT, AF>(W, gm, L, C, sp, op, row_of, sink);
  else
    walk_grouped<FMT>(W, gm, L, C, sp, op, row_of, sink);
}

template <int RF, int SF, int AF>
__global__ void __launch_bounds__(kBlock, 2) ggateup_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  ExpertLds L = carve(a, smem);
  const bool shared = (int)blockIdx.x < a.sh_wgs;
  const GroupMap& gm = shared ? a.sgm : a.rgm;
  const ClassCost k{gm.NG, gm.steps, gm.cw, gm.ct};
  Span sp;
  if (shared) {
    build_shared(a, L.sh, k.NG, k.steps, k.cw, k.ct);
    lds_barrier();
    sp = shared_span(a.T, k, gm.NS, blockIdx.x, a.sh_wgs, ShareW{0, a.ncu, a.late16});
  } else {
    build_routed(a, L, L.rt, k, gm.NS, blockIdx.x - a.sh_wgs, gridDim.x - a.sh_wgs);
    build_rows(a, L, L.rt);
    sp = read_span(L);
  }
  if (shared) ggateup_walk<SF, A_BF16>(a, L, L.sh, false, sp);
  else ggateup_walk<RF, AF>(a, L, L.rt, true, sp);
}

// =============================================================== grouped down kernel
// Row tile t: hidden rows [128 t, 128 t + 128), 32 per wave.
template <int FMT, int AF>
__device__ __forceinline__ void gdown_walk(const ExpertArgs& a, const ExpertLds& L, const ClassTab& C,
                                           bool routed, const Span& sp) {
  const WTensor& W = routed ? a.rw : a.sw;
  const GemvMap& m = routed ? a.rmap : a.smap;
  const GroupMap& gm = routed ? a.rgm : a.sgm;
  const DownOps<AF> op{a.h, a.hq_codes, a.hq_scales, a.hq_scale, W.gscale, W.gs_per_expert, W.rows,
                       routed ? a.I : a.Ish, m.RS, a.H, a.hs, a.o, L.w_tsc, C.r_pair, 1};
  const int wave = threadIdx.x / kWave, half = (threadIdx.x & (kWave - 1)) >> 5, lr = threadIdx.x & 31;
  auto row_of = [&](int e, int t, int r) -> int64_t { return (int64_t)e * W.rows + 128 * t + 32 * wave + r; };
  auto sink = [&](const UnitCtx& cx, int t, const f32x16_t& acc, float ts, float g, float) {
    if (lr >= cx.n) return;
    float* o = a.o + (int64_t)C.r_pair[cx.crow + lr] * a.H + 128 * t + 32 * wave;
    const float sc = g * ts;
#pragma unroll
    for (int r = 0; r < 16; ++r) o[acc_row(r, half)] = acc[r] * sc;
  };
  if constexpr (use_scaled_mfma<FMT, AF>())
    walk_grouped_mx<FMT, AF>(W, gm, L, C, sp, op, row_of, sink);
  else
    walk_grouped<FMT>(W, gm, L, C, sp, op, row_of, sink);   // h as BF16 (or its decoded codes)
}

template <int RF, int SF, int AF>
__global__ void __launch_bounds__(kBlock, 2) gdown_kernel(ExpertArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  ExpertLds L = carve(a, smem);
  const bool shared = (int)blockIdx.x < a.sh_wgs;
  const GroupMap& gm = shared ? a.sgm : a.rgm;
  const ClassCost k{gm.NG, gm.steps, gm.cw, gm.ct};
  Span sp;
  if (shared) {
    build_shared(a, L.sh, k.NG, k.steps, k.cw, k.ct);
    lds_barrier();
    sp = shared_span(a.T, k, gm.NS, blockIdx.x, a.sh_wgs, ShareW{0, a.ncu, a.late16});
  } else {
    build_routed(a, L, L.rt, k, gm.NS, blockIdx.x - a.sh_wgs, gridDim.x - a.sh_wgs);
    build_rows(a, L, L.rt);
    sp = read_span(L);
  }
  if (shared) gdown_walk<SF, A_BF16>(a, L, L.sh, false, sp);
  else gdown_walk<RF, AF>(a, L, L.rt, true, sp);
}

}  // namespace moe
