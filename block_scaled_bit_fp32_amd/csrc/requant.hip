// Load-time weight requantization (off the decode path). MXFP4 (and MXFP8 with E4M3
// elements, exponent offset 8 and saturation at 448): BF16 rows to E2M1
// values with one E8M0 scale per 32 (the Mistral Large 4 page's ROCm load path requantizes
// each expert this way, one layer at a time). The scale follows the OCP MX v1.0 rule:
// shared exponent floor(log2(block amax)) - 2, clamped to [-127, 127]; elements are the
// values times 2^-exponent (exact), rounded to E2M1 with ties to even and saturation at
// 6; an all-zero block takes exponent -127 and signed zero codes. NVFP4: the two-level
// recipe, one FP32 scale per tensor g = amax / 2688 and per 16-block the Four-Over-Six
// arithmetic with the target 6 only (E4M3 block scale (m / g) / 6, elements x / (S g)).
#include "launch.hpp"
#include "device.hpp"
#include "rows.hpp"

namespace moe {

// One thread per 32-element block; blocks are contiguous (cols % 32 == 0), so block b's
// 16 code bytes start at 16 b and its scale byte is b.
__global__ void __launch_bounds__(kBlock) requant_mxfp4_kernel(const uint16_t* x, int64_t nblocks, uint8_t* codes,
                                                               uint8_t* scales) {
  const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 r = src[q];
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      v[8 * q + 2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // floor(log2(amax)) = frexp exponent - 1 (amax = m * 2^e, m in [0.5, 1)), then - 2
  int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 3 : -127;
  e = min(max(e, -127), 127);
  // the hardware convert: two elements over the scale 2^e per instruction
  const float sc = __builtin_bit_cast(float, (uint32_t)(e + 127) << 23 | (e == -127 ? 0x00400000u : 0u));
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t r = 0u;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 0], v[8 * q + 1], sc, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 2], v[8 * q + 3], sc, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 4], v[8 * q + 5], sc, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * q + 6], v[8 * q + 7], sc, 3);
    w[q] = r;
  }
  *reinterpret_cast<uint4*>(codes + 16 * b) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[b] = (uint8_t)(e + 127);
}

// One workgroup per tensor of n elements (n % 16 == 0): the tensor's amax, then every
// 16-block with the c = 6 candidate.
__global__ void __launch_bounds__(kBlock) requant_nvfp4_kernel(const uint16_t* x, int64_t n, uint8_t* codes,
                                                               uint8_t* scales, float* gscale) {
  __shared__ float red[kBlock / kWave];
  const int64_t t = blockIdx.x, nb = n / 16;
  const Bf16Row row{x + t * n};
  float amax = 0.0f;
  for (int64_t b = threadIdx.x; b < nb; b += kBlock) {
    float v[16];
    row.load((int)b, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = block_max(amax, red);
  const float g = amax / 2688.0f;
  uint8_t* ct = codes + t * (n / 2);
  uint8_t* st = scales + t * nb;
  for (int64_t b = threadIdx.x; b < nb; b += kBlock) {
    float v[16];
    row.load((int)b, v);
    uint32_t sb = 0, c[2] = {0u, 0u};
    if (amax == 0.0f) {
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i >> 3] |= ((__float_as_uint(v[i]) >> 28) & 8u) << (4 * (i & 7));
    } else {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
      nvfp4_candidate(v, m, g, 6.0f, sb, c);
    }
    *reinterpret_cast<uint2*>(ct + 8 * b) = make_uint2(c[0], c[1]);
    st[b] = (uint8_t)sb;
  }
  if (threadIdx.x == 0) gscale[t] = g;
}

hipError_t launch_requant_nvfp4(const uint16_t* x, int ntensors, int64_t n, uint8_t* codes, uint8_t* scales,
                                float* gscale, hipStream_t s) {
  return launch_kernel(K_QUANT, requant_nvfp4_kernel, dim3(ntensors), dim3(kBlock), 0, s, x, n, codes, scales,
                       gscale);
}

// MXFP8: the same rule with the E4M3 element (largest exponent 8), one thread per
// 32-element block: 32 code bytes at 32 b, scale byte b.
__global__ void __launch_bounds__(kBlock) requant_mxfp8_kernel(const uint16_t* x, int64_t nblocks, uint8_t* codes,
                                                               uint8_t* scales) {
  const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (b >= nblocks) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + b * 32);
  float v[32];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint4 r = src[q];
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
      v[8 * q + 2 * i + 1] = bf16_to_f32(w[i] >> 16);
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 9 : -127;
  e = min(max(e, -127), 127);
  uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const float y = ldexpf(v[i], -e);
    w[i >> 2] |= (e4m3_encode_pos(fabsf(y)) | ((__float_as_uint(y) >> 24) & 0x80u)) << (8 * (i & 3));
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + 32 * b);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[b] = (uint8_t)(e + 127);
}

hipError_t launch_requant_mxfp8(const uint16_t* x, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                                hipStream_t s) {
  const int64_t grid = (nblocks + kBlock - 1) / kBlock;
  return launch_kernel(K_QUANT, requant_mxfp8_kernel, dim3((unsigned)grid), dim3(kBlock), 0, s, x, nblocks, codes,
                       scales);
}

hipError_t launch_requant_mxfp4(const uint16_t* x, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                                hipStream_t s) {
  const int64_t grid = (nblocks + kBlock - 1) / kBlock;
  return launch_kernel(K_QUANT, requant_mxfp4_kernel, dim3((unsigned)grid), dim3(kBlock), 0, s, x, nblocks, codes,
                       scales);
}

}  // namespace moe
