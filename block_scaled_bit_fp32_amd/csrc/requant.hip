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
  uint32_t w[4];
  const uint32_t sb = mx_block_fp4(v, w);
  *reinterpret_cast<uint4*>(codes + 16 * b) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[b] = (uint8_t)sb;
}

// NVFP4 in three launches over tensors of n elements (n % 16 == 0), in stream order, so
// no launch waits on another inside it:
//   1. grid (chunks, tensors): each workgroup's maximum |x| over kNvChunk elements, kept
//      as an FP32 in the tensor's code bytes (which launch 3 overwrites);
//   2. one workgroup per tensor: amax over those maxima (exact), g = amax / 2688;
//   3. grid (chunks, tensors): every 16-block of the chunk with the c = 6 candidate.
constexpr int kNvChunk = 16 * kBlock * 8;   // elements per workgroup (8 blocks of 16 per thread)

__global__ void __launch_bounds__(kBlock) nvfp4_chunk_max_kernel(const uint16_t* x, int64_t n, uint8_t* codes) {
  __shared__ float red[kBlock / kWave];
  const int64_t t = blockIdx.y, c = blockIdx.x;
  const int64_t b0 = c * (kNvChunk / 16), b1 = min(b0 + kNvChunk / 16, n / 16);
  const Bf16Row row{x + t * n};
  float amax = 0.0f;
  for (int64_t b = b0 + threadIdx.x; b < b1; b += kBlock) {
    float v[16];
    row.load((int)b, v);
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  }
  amax = block_max(amax, red);
  if (threadIdx.x == 0) reinterpret_cast<float*>(codes + t * (n / 2))[c] = amax;
}

__global__ void __launch_bounds__(kBlock) nvfp4_tensor_scale_kernel(const uint8_t* codes, int64_t n, int nchunks,
                                                                    float* gscale) {
  __shared__ float red[kBlock / kWave];
  const int64_t t = blockIdx.x;
  const float* part = reinterpret_cast<const float*>(codes + t * (n / 2));
  float amax = 0.0f;
  for (int c = threadIdx.x; c < nchunks; c += kBlock) amax = fmaxf(amax, part[c]);
  amax = block_max(amax, red);
  if (threadIdx.x == 0) gscale[t] = amax / 2688.0f;
}

// The c = 6 candidate of one 16-block (the scale and codes of nvfp4_candidate, in the same
// FP32 operation order, without its error sum).
__device__ __forceinline__ void nvfp4_block6(const float (&x)[16], float m, float g, uint32_t& sbyte,
                                             uint32_t (&codes)[2]) {
#pragma clang fp contract(off)
  const float u = (m / g) / 6.0f;
  sbyte = e4m3_encode_pos(u);
  const float d = e4m3_to_f32(sbyte) * g;
  codes[0] = codes[1] = 0u;
  if (d == 0.0f) {
#pragma unroll
    for (int i = 0; i < 16; ++i) codes[i >> 3] |= ((__float_as_uint(x[i]) >> 28) & 8u) << (4 * (i & 7));
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) codes[i >> 3] |= e2m1_encode(x[i] / d) << (4 * (i & 7));
  }
}

__global__ void __launch_bounds__(kBlock) nvfp4_quant_kernel(const uint16_t* x, int64_t n, uint8_t* codes,
                                                             uint8_t* scales, const float* gscale) {
  const int64_t t = blockIdx.y, c = blockIdx.x;
  const int64_t b0 = c * (kNvChunk / 16), b1 = min(b0 + kNvChunk / 16, n / 16);
  const Bf16Row row{x + t * n};
  const float g = gscale[t];
  uint8_t* ct = codes + t * (n / 2);
  uint8_t* st = scales + t * (n / 16);
  for (int64_t b = b0 + threadIdx.x; b < b1; b += kBlock) {
    float v[16];
    row.load((int)b, v);
    uint32_t sb = 0, cw[2] = {0u, 0u};
    if (g == 0.0f) {   // all-zero tensor (amax / 2688 is zero only for amax = 0)
#pragma unroll
      for (int i = 0; i < 16; ++i) cw[i >> 3] |= ((__float_as_uint(v[i]) >> 28) & 8u) << (4 * (i & 7));
    } else {
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
      nvfp4_block6(v, m, g, sb, cw);
    }
    *reinterpret_cast<uint2*>(ct + 8 * b) = make_uint2(cw[0], cw[1]);
    st[b] = (uint8_t)sb;
  }
}

hipError_t launch_requant_nvfp4(const uint16_t* x, int ntensors, int64_t n, uint8_t* codes, uint8_t* scales,
                                float* gscale, hipStream_t s) {
  const int64_t nchunks = (n + kNvChunk - 1) / kNvChunk;
  const dim3 grid((unsigned)nchunks, (unsigned)ntensors);
  hipError_t err = launch_kernel(K_QUANT, nvfp4_chunk_max_kernel, grid, dim3(kBlock), 0, s, x, n, codes);
  if (err != hipSuccess) return err;
  err = launch_kernel(K_QUANT, nvfp4_tensor_scale_kernel, dim3(ntensors), dim3(kBlock), 0, s,
                      (const uint8_t*)codes, n, (int)nchunks, gscale);
  if (err != hipSuccess) return err;
  return launch_kernel(K_QUANT, nvfp4_quant_kernel, grid, dim3(kBlock), 0, s, x, n, codes, scales,
                       (const float*)gscale);
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
  uint32_t w[8];
  const uint32_t sb = mx_block_fp8(v, w);
  uint4* dst = reinterpret_cast<uint4*>(codes + 32 * b);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[b] = (uint8_t)sb;
}

// Block-scaled FP8 input (the checkpoint the Mistral Large 4 page's loader reads: E4M3
// expert weights with one FP32 scale per block_rows x block_cols block): each value is
// decoded, multiplied by its block's scale (one FP32 product) and rounded to BF16, the
// expert's BF16 form; its 32-blocks then take the MXFP4 rule above. One thread per
// 32-block of a row: block b holds row r = b / (cols / 32), columns c0 .. c0 + 31, whose
// scales sit in row r / block_rows of the scale grid, from column c0 / block_cols on.
__global__ void __launch_bounds__(kBlock) requant_fp8b_mxfp4_kernel(const uint8_t* w, const float* bscale,
                                                                    int64_t nblocks, int cols, int block_rows,
                                                                    int block_cols, int scale_cols, uint8_t* codes,
                                                                    uint8_t* scales) {
  const int64_t b = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (b >= nblocks) return;
  const int per_row = cols / 32;
  const int64_t r = b / per_row;
  const int c0 = (int)(b - r * per_row) * 32;
  const float* srow = bscale + (r / block_rows) * scale_cols;
  const uint4* src = reinterpret_cast<const uint4*>(w + b * 32);
  const uint4 q0 = src[0], q1 = src[1];
  const uint32_t wd[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
  int sc = c0 / block_cols;
  int next = (sc + 1) * block_cols;   // first column of the next scale block
  float s = srow[sc];
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    if (c0 + i == next) {
      ++sc;
      next += block_cols;
      s = srow[sc];
    }
    const float p = e4m3_to_f32((wd[i >> 2] >> (8 * (i & 3))) & 0xFFu) * s;
    v[i] = bf16_to_f32(f32_to_bf16_rne(p));
  }
  uint32_t q[4];
  const uint32_t sb = mx_block_fp4(v, q);
  *reinterpret_cast<uint4*>(codes + 16 * b) = make_uint4(q[0], q[1], q[2], q[3]);
  scales[b] = (uint8_t)sb;
}

hipError_t launch_requant_fp8b_mxfp4(const uint8_t* w, const float* bscale, int64_t rows, int cols, int block_rows,
                                     int block_cols, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t nblocks = rows * (cols / 32);
  const int64_t grid = (nblocks + kBlock - 1) / kBlock;
  const int scale_cols = (cols + block_cols - 1) / block_cols;
  return launch_kernel(K_QUANT, requant_fp8b_mxfp4_kernel, dim3((unsigned)grid), dim3(kBlock), 0, s, w, bscale,
                       nblocks, cols, block_rows, block_cols, scale_cols, codes, scales);
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
