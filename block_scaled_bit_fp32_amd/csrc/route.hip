// Router GEMV and top-k (two launches: the top-k needs every logit of a token),
// token quantization, the standalone Four-Over-Six quantizer and the workspace fill
// kernel.
#include <algorithm>
#include <type_traits>

#include "launch.hpp"
#include "rows.hpp"
#include "topk.hpp"

namespace moe {

// ===================================================================== quantize
__global__ void __launch_bounds__(kBlock)
quantize_nvfp4_kernel(const uint16_t* x, int cols, uint8_t* codes, uint8_t* scales, float* g,
                      uint8_t* choice) {
  __shared__ float red[kBlock / kWave];
  const int r = blockIdx.x;
  quant_row_nvfp4(Bf16Row{x + (int64_t)r * cols}, cols, codes + (int64_t)r * (cols / 2),
                  scales + (int64_t)r * (cols / 16), g + r,
                  choice ? choice + (int64_t)r * (cols / 16) : nullptr, red);
}

// Quantizes token t's row (BF16 tokens, or the normalized ones) per the layer's
// activation format; BF16 layers quantize nothing.
template <class Row>
__device__ __forceinline__ void quant_token(const RouteArgs& a, const Row& row, int t, float* red) {
  if (a.afmt == A_NVFP4_4O6) {
    quant_row_nvfp4(row, a.H, a.xq_codes + (int64_t)t * (a.H / 2), a.xq_scales + (int64_t)t * (a.H / 16),
                    a.xq_scale + t, nullptr, red);
  } else if (a.afmt == A_FP8_TOKEN) {
    quant_row_fp8(row, a.H, a.xq_codes + (int64_t)t * a.H, a.xq_scale + t, red);
  } else if (a.afmt == A_MXFP4) {
    quant_row_mx<false>(row, a.H, a.xq_codes + (int64_t)t * (a.H / 2), a.xq_scales + (int64_t)t * (a.H / 32));
  } else if (a.afmt == A_MXFP8) {
    quant_row_mx<true>(row, a.H, a.xq_codes + (int64_t)t * a.H, a.xq_scales + (int64_t)t * (a.H / 32));
  }
}

// ======================================================================== route
// Router GEMV: workgroups tile (tokens x experts); each of the 4 waves reduces a quarter
// of H, the partial sums meet in LDS in a fixed order. Extra workgroups (one per token)
// quantize the tokens in the same launch when the layer quantizes x (Four-Over-Six
// NVFP4, FP8 per token, MXFP4 or MXFP8). NORM: the layer's input is the RMSNorm of the
// residual stream (rows.hpp); the router workgroups compute each token's normalized
// values on the fly and the per-token workgroups write them (the same bits: the same
// code in the same order) and quantize them.
template <int ET, int TT, bool NORM>
__global__ void __launch_bounds__(kBlock) route_gemv_kernel(RouteArgs a) {
  warm_args<RouteArgs>();
  __shared__ float red[(kBlock / kWave) * ET * TT];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n_router = a.n_tt * a.n_et;
  if ((int)blockIdx.x >= n_router) {  // per-token workgroups
    const int t = blockIdx.x - n_router;
    if constexpr (NORM) {
      const uint16_t* r = a.resid + (int64_t)t * a.H;
      const float rstd = row_rstd(r, a.H, a.eps, red);
      const NormRow row{r, a.gamma, rstd};
      for (int c = threadIdx.x; c < a.H / 16; c += kBlock) {   // x: 16 elements per step
        float v[16];
        row.load(c, v);
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = (__float_as_uint(v[2 * i]) >> 16) | (__float_as_uint(v[2 * i + 1]) & 0xFFFF0000u);
        uint4* dst = reinterpret_cast<uint4*>(a.x_out + (int64_t)t * a.H + 16 * c);
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      }
      quant_token(a, row, t, red);
    } else {
      quant_token(a, Bf16Row{a.x + (int64_t)t * a.H}, t, red);
    }
    return;
  }
  const int tt = blockIdx.x / a.n_et, et = blockIdx.x % a.n_et;
  const int t0 = tt * TT, e0 = et * ET;
  const int nt = min(TT, a.T - t0), ne = min(ET, a.E - e0);
  const int quarter = a.H / 4;        // elements of K per wave
  const int kb = wave * quarter;
  float rstd[TT];
  if constexpr (NORM) {
#pragma unroll
    for (int t = 0; t < TT; ++t) rstd[t] = row_rstd(a.resid + (int64_t)(t0 + min(t, nt - 1)) * a.H, a.H, a.eps, red);
    __syncthreads();   // every wave has read the last sum before red holds partial logits
  }
  float acc[ET][TT];
#pragma unroll
  for (int e = 0; e < ET; ++e)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[e][t] = 0.0f;
  // Rows past the tile's last expert or token re-read its last one (results unused), so
  // every load of an iteration issues before the first use.
#pragma unroll 2
  for (int c = lane * 4; c < quarter; c += kWave * 4) {
    const int h = kb + c;
    float4 wv[ET];
    uint2 xb[TT];
    uint2 gb = make_uint2(0u, 0u);
#pragma unroll
    for (int e = 0; e < ET; ++e)
      wv[e] = *reinterpret_cast<const float4*>(a.wr + (int64_t)(e0 + min(e, ne - 1)) * a.H + h);
#pragma unroll
    for (int t = 0; t < TT; ++t)
      xb[t] = *reinterpret_cast<const uint2*>((NORM ? a.resid : a.x) + (int64_t)(t0 + min(t, nt - 1)) * a.H + h);
    if constexpr (NORM) gb = *reinterpret_cast<const uint2*>(a.gamma + h);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      float x0 = bf16_to_f32(xb[t].x & 0xFFFFu), x1 = bf16_to_f32(xb[t].x >> 16);
      float x2 = bf16_to_f32(xb[t].y & 0xFFFFu), x3 = bf16_to_f32(xb[t].y >> 16);
      if constexpr (NORM) {
        x0 = norm_x(x0, rstd[t], bf16_to_f32(gb.x & 0xFFFFu));
        x1 = norm_x(x1, rstd[t], bf16_to_f32(gb.x >> 16));
        x2 = norm_x(x2, rstd[t], bf16_to_f32(gb.y & 0xFFFFu));
        x3 = norm_x(x3, rstd[t], bf16_to_f32(gb.y >> 16));
      }
#pragma unroll
      for (int e = 0; e < ET; ++e)
        acc[e][t] = fmaf(wv[e].w, x3, fmaf(wv[e].z, x2, fmaf(wv[e].y, x1, fmaf(wv[e].x, x0, acc[e][t]))));
    }
  }
#pragma unroll
  for (int e = 0; e < ET; ++e)
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t < nt) {
        const float v = group_sum<kWave>(acc[e][t]);
        if (lane == 0) red[(wave * ET + e) * TT + t] = v;
      }
    }
  __syncthreads();
  if ((int)threadIdx.x < ET * TT) {
    const int e = threadIdx.x / TT, t = threadIdx.x % TT;
    if (e < ne && t < nt) {
      float v = red[(0 * ET + e) * TT + t];
#pragma unroll
      for (int w = 1; w < kBlock / kWave; ++w) v += red[(w * ET + e) * TT + t];
      if (a.raw) a.raw[(int64_t)(t0 + t) * a.E + e0 + e] = v;
      if (a.bias) v += a.bias[e0 + e];
      a.logits[(int64_t)(t0 + t) * a.E + e0 + e] = v;
    }
  }
}

// Top-k: one wave per token (wave_topk).
template <int NK>
__global__ void __launch_bounds__(kBlock) topk_kernel(RouteArgs a) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave;
  if (t >= a.T) return;
  int e;
  float w;
  wave_topk<NK>(a.logits + (int64_t)t * a.E, a.E, a.k, a.raw ? a.raw + (int64_t)t * a.E : nullptr, a.softmax, e, w);
  if (lane < a.k) {
    a.ids[(int64_t)t * a.k + lane] = e;
    a.w[(int64_t)t * a.k + lane] = w;
  }
}

// ================================================================ host launchers
__global__ void fill_zero_kernel(uint4* p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int grid = (int)std::min<int64_t>(1024, (n16 + kBlock - 1) / kBlock);
  if (grid <= 0) return hipSuccess;
  return launch_kernel(K_FILL, fill_zero_kernel, dim3(grid), dim3(kBlock), 0, s, (uint4*)p, n16);
}

hipError_t launch_quantize_nvfp4(const uint16_t* x, int rows, int cols, uint8_t* codes, uint8_t* scales,
                                 float* g, uint8_t* choice, hipStream_t s) {
  return launch_kernel(K_QUANT, quantize_nvfp4_kernel, dim3(rows), dim3(kBlock), 0, s, x, cols, codes,
                       scales, g, choice);
}

hipError_t launch_route(const RouteArgs& a, int n_quant, bool topk, hipStream_t s) {
  const int grid = a.n_tt * a.n_et + n_quant;
  auto go = [&](auto kern) { return launch_kernel(K_ROUTE, kern, dim3(grid), dim3(kBlock), 0, s, a); };
  // tiles the host picks: one token (1, 2 or 4 experts), or 8 tokens x 4 experts
  auto pick = [&](auto norm) {
    constexpr bool N = decltype(norm)::value;
    return a.TT == 8 ? go(route_gemv_kernel<4, 8, N>)
           : a.ET == 1 ? go(route_gemv_kernel<1, 1, N>)
           : a.ET == 2 ? go(route_gemv_kernel<2, 1, N>)
                       : go(route_gemv_kernel<4, 1, N>);
  };
  hipError_t err = a.resid ? pick(std::integral_constant<bool, true>{}) : pick(std::integral_constant<bool, false>{});
  if (err != hipSuccess || !topk) return err;
  const dim3 tg((a.T + kBlock / kWave - 1) / (kBlock / kWave));
  if (a.E <= 64) return launch_kernel(K_TOPK, topk_kernel<1>, tg, dim3(kBlock), 0, s, a);
  if (a.E <= 128) return launch_kernel(K_TOPK, topk_kernel<2>, tg, dim3(kBlock), 0, s, a);
  if (a.E <= 256) return launch_kernel(K_TOPK, topk_kernel<4>, tg, dim3(kBlock), 0, s, a);
  if (a.E <= 384) return launch_kernel(K_TOPK, topk_kernel<6>, tg, dim3(kBlock), 0, s, a);
  if (a.E <= 512) return launch_kernel(K_TOPK, topk_kernel<8>, tg, dim3(kBlock), 0, s, a);
  return launch_kernel(K_TOPK, topk_kernel<16>, tg, dim3(kBlock), 0, s, a);
}

}  // namespace moe
