// Device helpers for the gfx950 MoE kernels: format conversion, encoders, reductions.
//
// Formats (OCP Microscaling v1.0 bit layouts; the pages name NVFP4, MXFP4 and MXFP8 in
// "Inkling 2 Small on vLLM: Day-0 Support", mixed-precision MoE, and in "Day 0 support
// for Mistral Large 4 on vLLM", ROCm implementation details):
//   E2M1 nibble s|ee|m, values 0, .5, 1, 1.5, 2, 3, 4, 6;  E4M3 byte s|eeee|mmm, bias 7,
//   max 448, 0x7F/0xFF NaN;  E8M0 byte = 2^(b-127).
// gfx950 decodes E2M1 and E4M3 in hardware (v_cvt_scalef32_pk_*_fp4/_fp8, v_cvt_f32_fp8,
// OCP variants). The "scalef32" operand of those instructions only contributes its
// exponent, so it can carry an E8M0 scale exactly but not an E4M3 one.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 256;  // threads per workgroup in every kernel

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// FP32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  uint32_t b = __float_as_uint(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b == 0 ? __uint_as_float(0x00400000u) : __uint_as_float(b << 23);
}

__device__ __forceinline__ uint32_t as_u32(bf16x2_t v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); }

// Two E2M1 values from byte `sel` of w -> two BF16 (low nibble first), times 2^exp(scale).
template <int SEL>
__device__ __forceinline__ bf16x2_t fp4x2_to_bf16(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, SEL);
}
template <int SEL>
__device__ __forceinline__ f32x2_t fp4x2_to_f32(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, SEL);
}
// Two E4M3 values from 16-bit half `HI` of w.
template <bool HI>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, scale, HI);
}
template <bool HI>
__device__ __forceinline__ f32x2_t fp8x2_to_f32(uint32_t w, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, scale, HI);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load that should not displace reused data from the caches.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

// Marks a value that is the same on every lane (read from LDS, say) as wave-uniform,
// so that branches on it are scalar branches instead of exec-masked code.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// ---------------------------------------------------------------- barriers
// Workgroup barrier for LDS traffic only: waits for this wave's LDS operations, then
// for every wave. Unlike __syncthreads it does not wait for outstanding global loads,
// so weight loads already in flight keep streaming across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Brings every 64-byte line of a kernel's argument block (an Args struct passed by value)
// into the scalar cache at the kernel's start. The compiler loads the argument fields it
// needs in several batches (it keeps few in scalar registers and reloads them), each batch
// waiting for all of its loads; a batch that touches a line not cached yet waits a memory
// round trip, and several such batches in a row delay the prologue. One plain load per
// line, consumed together, joins the first batch, so later batches hit the cache.
// Offsets stay inside the struct.
template <class Args>
__device__ __forceinline__ void warm_args() {
  constexpr int S = (int)sizeof(Args);
  static_assert(S >= 4 && S <= 64 * 12, "argument block of at most 12 lines");
  const auto* p = (const __attribute__((address_space(4))) uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
  auto at = [&](int i) { return p[(64 * i < S - 4 ? 64 * i : S - 4) / 4]; };
  // one statement consumes every value, so the loads go out in one batch
  asm volatile("" ::"s"(at(0)), "s"(at(1)), "s"(at(2)), "s"(at(3)), "s"(at(4)), "s"(at(5)), "s"(at(6)),
               "s"(at(7)), "s"(at(8)), "s"(at(9)), "s"(at(10)), "s"(at(11)), "s"(p[S / 4 - 1]));
}

// ---------------------------------------------------------------- reductions
// Wave-wide maximum of a 64-bit key, returned to every lane. Within each row of 16
// lanes DPP moves (xor 1, xor 2, rotate 4, rotate 8) spread the row maximum to all its
// lanes; the four row maxima are then read out (readlane) and combined in scalars.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t k) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t k, int lane) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, lane);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), lane);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  uint64_t p;
  p = dpp_u64<0xB1>(k); k = p > k ? p : k;    // quad_perm [1,0,3,2]
  p = dpp_u64<0x4E>(k); k = p > k ? p : k;    // quad_perm [2,3,0,1]
  p = dpp_u64<0x124>(k); k = p > k ? p : k;   // row_ror:4
  p = dpp_u64<0x128>(k); k = p > k ? p : k;   // row_ror:8
  uint64_t r = readlane_u64(k, 0);
  p = readlane_u64(k, 16); r = p > r ? p : r;
  p = readlane_u64(k, 32); r = p > r ? p : r;
  p = readlane_u64(k, 48); r = p > r ? p : r;
  return r;
}

// The same for 32-bit values (maximum, and minimum), returned as a scalar.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_ext_u32(uint32_t k) {
  auto pick = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  k = pick(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  k = pick(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  k = pick(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x124, 0xF, 0xF, false));   // row_ror:4
  k = pick(k, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)k, 0x128, 0xF, 0xF, false));   // row_ror:8
  uint32_t r = (uint32_t)__builtin_amdgcn_readlane((int)k, 0);
  r = pick(r, (uint32_t)__builtin_amdgcn_readlane((int)k, 16));
  r = pick(r, (uint32_t)__builtin_amdgcn_readlane((int)k, 32));
  return pick(r, (uint32_t)__builtin_amdgcn_readlane((int)k, 48));
}

// Wave-wide inclusive prefix sum (lane i gets the sum over lanes 0..i). Within each row
// of 16 lanes, DPP row shifts by 1, 2, 4, 8 (lanes shifted in from outside the row add
// 0); then row_bcast:15 adds row 0's and row 2's totals to rows 1 and 3, and
// row_bcast:31 adds the total of rows 0-1 to rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add_src(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROWS, 0xF, false);
}
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += dpp_add_src<0x111, 0xF>(x);   // row_shr:1
  x += dpp_add_src<0x112, 0xF>(x);   // row_shr:2
  x += dpp_add_src<0x114, 0xF>(x);   // row_shr:4
  x += dpp_add_src<0x118, 0xF>(x);   // row_shr:8
  x += dpp_add_src<0x142, 0xA>(x);   // row_bcast:15 into rows 1, 3
  x += dpp_add_src<0x143, 0xC>(x);   // row_bcast:31 into rows 2, 3
  return x;
}

// Order-preserving map of a finite float to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Workgroup max of non-negative values (every thread gets the result). `red` holds
// kBlock / kWave floats of LDS.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kBlock / kWave; ++w) r = fmaxf(r, red[w]);
  return r;
}

// ---------------------------------------------------------------- encoders
// These define the quantizers bit for bit. The operation order is fixed and nothing
// may be contracted into an FMA: compile this code with FP contraction off.

// Non-negative finite u -> E4M3 byte, nearest with ties to even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_encode_pos(float u) {
  if (!(u < 448.0f)) return 0x7Eu;              // 448 and above (RNE then satfinite)
  if (u < 0x1p-6f) {                             // zero and subnormals: steps of 2^-9
    return (uint32_t)__builtin_rintf(u * 512.0f);  // exact scaling; 8 -> 0x08 = 2^-6
  }
  const uint32_t b = __float_as_uint(u);
  const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);  // round to 3 mantissa bits, even
  return (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u); // rebias 127 -> 7
}

// Finite y -> E2M1 code, nearest with ties to the even code, saturating at 6, sign
// copied from y (so -0 and small negatives give code 8).
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
  const float a = fabsf(y);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return m | ((__float_as_uint(y) >> 28) & 8u);
}

__device__ __forceinline__ float e2m1_magnitude(uint32_t m) {
  return m < 4u ? 0.5f * (float)m : (m < 7u ? (float)(m - 2u) : 6.0f);
}

// One Four-Over-Six candidate for a 16-element block x (FP32), block max m, row
// scale g > 0 and target c (6 or 4). Writes the scale byte and packed codes (8 bytes
// as two words, element 2i in the low nibble) and returns the FP32 error sum.
__device__ __forceinline__ float nvfp4_candidate(const float (&x)[16], float m, float g, float c,
                                                 uint32_t& sbyte, uint32_t (&codes)[2]) {
#pragma clang fp contract(off)
  const float u = (m / g) / c;
  sbyte = e4m3_encode_pos(u);
  const float S = e4m3_to_f32(sbyte);
  const float d = S * g;
  float e[16];
  codes[0] = codes[1] = 0u;
  if (d == 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      e[i] = fabsf(x[i]);
      codes[i >> 3] |= ((__float_as_uint(x[i]) >> 28) & 8u) << (4 * (i & 7));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t q = e2m1_encode(x[i] / d);
      const float mag = e2m1_magnitude(q & 7u) * d;
      const float r = (q & 8u) ? -mag : mag;
      e[i] = fabsf(x[i] - r);
      codes[i >> 3] |= q << (4 * (i & 7));
    }
  }
  // pairwise tree: (i, i+8), then (i, i+4), (i, i+2), (0, 1)
  float s8[8], s4[4], s2[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) s8[i] = e[i] + e[i + 8];
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = s8[i] + s8[i + 4];
#pragma unroll
  for (int i = 0; i < 2; ++i) s2[i] = s4[i] + s4[i + 2];
  return s2[0] + s2[1];
}

// Four-Over-Six for one block: returns the chosen target (4 or 6).
__device__ __forceinline__ uint32_t nvfp4_4o6_block(const float (&x)[16], float g, uint32_t& sbyte,
                                                    uint32_t (&codes)[2]) {
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(x[i]));
  uint32_t sb6, sb4, c6[2], c4[2];
  const float e6 = nvfp4_candidate(x, m, g, 6.0f, sb6, c6);
  const float e4 = nvfp4_candidate(x, m, g, 4.0f, sb4, c4);
  const bool four = e4 < e6;
  sbyte = four ? sb4 : sb6;
  codes[0] = four ? c4[0] : c6[0];
  codes[1] = four ? c4[1] : c6[1];
  return four ? 4u : 6u;
}

// OCP MX v1.0 of one 32-element block (the Mistral Large 4 page's MXFP4 load path and
// MX activations): shared exponent e = floor(log2(block amax)) - emax, emax the element
// format's largest exponent (E2M1: 2, E4M3: 8), clamped to [-127, 127] (an all-zero block
// takes -127); elements are the values times 2^-e (exact), rounded to the element
// format with ties to even and saturation, sign kept. Returns the E8M0 scale byte e + 127.
// E2M1: gfx950's scaled FP32 -> FP4 convert does the scaling and rounding, two
// elements per instruction; codes in w[4] (element 2i in the low nibble).
__device__ __forceinline__ uint32_t mx_block_fp4(const float (&v)[32], uint32_t (&w)[4]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // floor(log2(amax)) = frexp exponent - 1 (amax = m * 2^e, m in [0.5, 1)), then - 2
  int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 3 : -127;
  e = min(max(e, -127), 127);
  const float sc = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23 | (e == -127 ? 0x00400000u : 0u));
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t r = 0u;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 0], v[8 * q + 1], sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 2], v[8 * q + 3], sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 4], v[8 * q + 5], sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 6], v[8 * q + 7], sc, 3);
    w[q] = r;
  }
  return (uint32_t)(e + 127);
}

// The same with E4M3 elements (largest exponent 8, saturation at 448): codes in w[8].
__device__ __forceinline__ uint32_t mx_block_fp8(const float (&v)[32], uint32_t (&w)[8]) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 9 : -127;
  e = min(max(e, -127), 127);
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = 0u;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float y = ldexpf(v[i], -e);
    w[i >> 2] |= (e4m3_encode_pos(fabsf(y)) | ((__float_as_uint(y) >> 24) & 0x80u)) << (8 * (i & 3));
  }
  return (uint32_t)(e + 127);
}

// FP8-E4M3 of x / s (finite), sign copied from x.
__device__ __forceinline__ uint32_t fp8_token_code(float x, float s) {
#pragma clang fp contract(off)
  const float y = x / s;
  return e4m3_encode_pos(fabsf(y)) | ((__float_as_uint(y) >> 24) & 0x80u);
}

}  // namespace moe
