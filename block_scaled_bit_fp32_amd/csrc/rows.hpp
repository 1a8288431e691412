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
