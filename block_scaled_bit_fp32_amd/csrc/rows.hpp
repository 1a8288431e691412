// Whole-workgroup row quantizers shared by the route, expert and standalone kernels.
#pragma once
#include "device.hpp"
#include "plan.hpp"

namespace moe {

// =========================================================================== rows
struct Bf16Row {
  const uint16_t* p;
  __device__ __forceinline__ void load(int b, float (&v)[16]) const {
    const uint4* q = reinterpret_cast<const uint4*>(p + 16 * b);
    const uint4 a = q[0], c = q[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      v[2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
};

struct F32Row {
  const float* p;
  __device__ __forceinline__ void load(int b, float (&v)[16]) const {
    const float4* q = reinterpret_cast<const float4*>(p + 16 * b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = q[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  }
};

// ----------------------------------------------------------------- RMSNorm
// The MoE sublayer's input as the RMSNorm of the residual stream ("Day 0 support for
// Mistral Large 4 on vLLM", decode-round fusions: residual add and RMSNorm in one kernel;
// "Inkling 2 Small on vLLM: Day-0 Support", kernel fusion of the memory-bound steps
// between sublayers): x = r / sqrt(mean(r^2) + eps) * gamma, rounded to BF16. In FP32 in a
// fixed order, so every workgroup that needs a token's x computes the same bits: thread i
// sums the squares of elements i, i + kBlock, ...; the wave sums them in an xor tree, and
// the four waves' sums are added in wave order.
__device__ __forceinline__ float block_sum_fixed(float v, float* red) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}
__device__ __forceinline__ float row_rstd(const uint16_t* r, int H, float eps, float* red) {
#pragma clang fp contract(off)
  float ss = 0.0f;
  for (int h = threadIdx.x; h < H; h += kBlock) {
    const float v = bf16_to_f32(r[h]);
    ss = ss + v * v;
  }
  ss = block_sum_fixed(ss, red);
  return 1.0f / sqrtf(ss / (float)H + eps);
}
// One normalized element, rounded to BF16 (returned as its FP32 value).
__device__ __forceinline__ float norm_x(float r, float rstd, float g) {
#pragma clang fp contract(off)
  const float v = (r * rstd) * g;
  return bf16_to_f32(f32_to_bf16_rne(v));
}
// Rows of normalized tokens for the quantizers: 16 elements at a time.
struct NormRow {
  const uint16_t* r;
  const uint16_t* g;
  float rstd;
  __device__ __forceinline__ void load(int b, float (&v)[16]) const {
    const uint4* q = reinterpret_cast<const uint4*>(r + 16 * b);
    const uint4* w = reinterpret_cast<const uint4*>(g + 16 * b);
    const uint4 a = q[0], c = q[1], ga = w[0], gc = w[1];
    const uint32_t x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
    const uint32_t y[8] = {ga.x, ga.y, ga.z, ga.w, gc.x, gc.y, gc.z, gc.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = norm_x(bf16_to_f32(x[i] & 0xFFFFu), rstd, bf16_to_f32(y[i] & 0xFFFFu));
      v[2 * i + 1] = norm_x(bf16_to_f32(x[i] >> 16), rstd, bf16_to_f32(y[i] >> 16));
    }
  }
};

// Four-Over-Six NVFP4 of one row of n elements (n % 16 == 0), whole workgroup.
template <class Row>
__device__ __forceinline__ void quant_row_nvfp4(const Row& row, int n, uint8_t* codes, uint8_t* scales,
                                float* gout, uint8_t* choice, float* red) {
  const int nb = n >> 4;
  float amax = 0.0f;
  for (int b = threadIdx.x; b < nb; b += kBlock) {
    float v[16];
    row.load(b, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = block_max(amax, red);
  const float g = amax / 2688.0f;
  for (int b = threadIdx.x; b < nb; b += kBlock) {
    float v[16];
    row.load(b, v);
    uint32_t sb = 0, c[2] = {0u, 0u}, ch = 6;
    if (amax == 0.0f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i >> 3] |= ((__float_as_uint(v[i]) >> 28) & 8u) << (4 * (i & 7));
    } else {
      ch = nvfp4_4o6_block(v, g, sb, c);
    }
    *reinterpret_cast<uint2*>(codes + 8 * b) = make_uint2(c[0], c[1]);
    scales[b] = (uint8_t)sb;
    if (choice) choice[b] = (uint8_t)ch;
  }
  if (threadIdx.x == 0) *gout = g;
}

// FP8-E4M3 with one FP32 scale amax/448 for one row of n elements (n % 16 == 0).
template <class Row>
__device__ __forceinline__ void quant_row_fp8(const Row& row, int n, uint8_t* codes, float* sout, float* red) {
  const int nb = n >> 4;
  float amax = 0.0f;
  for (int b = threadIdx.x; b < nb; b += kBlock) {
    float v[16];
    row.load(b, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = block_max(amax, red);
  const float s = amax / 448.0f;
  for (int b = threadIdx.x; b < nb; b += kBlock) {
    float v[16];
    row.load(b, v);
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t q = amax == 0.0f ? ((__float_as_uint(v[i]) >> 24) & 0x80u) : fp8_token_code(v[i], s);
      w[i >> 2] |= q << (8 * (i & 3));
    }
    *reinterpret_cast<uint4*>(codes + 16 * b) = make_uint4(w[0], w[1], w[2], w[3]);
  }
  if (threadIdx.x == 0) *sout = s;
}

// OCP MX (MXFP4 or MXFP8) of one row of n elements (n % 32 == 0), whole workgroup: one
// thread per 32-block (mx_block_fp4 / mx_block_fp8). Codes [n/2] or [n] bytes, E8M0
// scales [n/32]. Blocks are independent: no row-wide reduction.
template <bool FP8, class Row>
__device__ __forceinline__ void quant_row_mx(const Row& row, int n, uint8_t* codes, uint8_t* scales) {
  const int nb = n >> 5;
  for (int b = threadIdx.x; b < nb; b += kBlock) {
    float v[32], lo[16], hi[16];
    row.load(2 * b, lo);
    row.load(2 * b + 1, hi);
#pragma unroll
    for (int i = 0; i < 16; ++i) { v[i] = lo[i]; v[16 + i] = hi[i]; }
    if constexpr (FP8) {
      uint32_t w[8];
      scales[b] = (uint8_t)mx_block_fp8(v, w);
      uint4* dst = reinterpret_cast<uint4*>(codes + 32 * b);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      uint32_t w[4];
      scales[b] = (uint8_t)mx_block_fp4(v, w);
      *reinterpret_cast<uint4*>(codes + 16 * b) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

}  // namespace moe
