// Kernels between and after the expert GEMVs:
//   hquant_kernel   re-quantizes each routed pair's SwiGLU output h (FP32, one row of I)
//                   per the layer's activation format (Four-Over-Six NVFP4, FP8 per row,
//                   MXFP4 or MXFP8 per 32-block) -- the quantize-before-down step of the
//                   Inkling page's MoE with fused activation quantization, once per pair.
//   combine_kernel  y[t][r] = sum_j w[t][j] * o[t*k+j][r] (+ o_shared[t][r]) (+ the residual
//                   stream's r[t][r]), FP32 in that order, rounded to BF16 -- the weighted
//                   combine (k <= 16).
#include "launch.hpp"
#include "rows.hpp"

namespace moe {

__global__ void __launch_bounds__(kBlock) hquant_kernel(ExpertArgs a) {
  __shared__ float red[kBlock / kWave];
  const int p = blockIdx.x;   // pair t*k + j
  const F32Row row{a.h + (int64_t)p * a.hs};
  if (a.afmt == A_NVFP4_4O6) {
    quant_row_nvfp4(row, a.I, a.hq_codes + (int64_t)p * (a.I / 2), a.hq_scales + (int64_t)p * (a.I / 16),
                    a.hq_scale + p, nullptr, red);
    if (a.dbg_codes)
      quant_row_nvfp4(row, a.I, a.dbg_codes + (int64_t)p * (a.I / 2), a.dbg_scales + (int64_t)p * (a.I / 16),
                      a.dbg_scale + p, nullptr, red);
  } else if (a.afmt == A_FP8_TOKEN) {
    quant_row_fp8(row, a.I, a.hq_codes + (int64_t)p * a.I, a.hq_scale + p, red);
    if (a.dbg_codes) quant_row_fp8(row, a.I, a.dbg_codes + (int64_t)p * a.I, a.dbg_scale + p, red);
  } else if (a.afmt == A_MXFP4) {
    quant_row_mx<false>(row, a.I, a.hq_codes + (int64_t)p * (a.I / 2), a.hq_scales + (int64_t)p * (a.I / 32));
    if (a.dbg_codes)
      quant_row_mx<false>(row, a.I, a.dbg_codes + (int64_t)p * (a.I / 2), a.dbg_scales + (int64_t)p * (a.I / 32));
  } else {
    quant_row_mx<true>(row, a.I, a.hq_codes + (int64_t)p * a.I, a.hq_scales + (int64_t)p * (a.I / 32));
    if (a.dbg_codes)
      quant_row_mx<true>(row, a.I, a.dbg_codes + (int64_t)p * a.I, a.dbg_scales + (int64_t)p * (a.I / 32));
  }
}

// One thread per (token, hidden row); grid (ceil(H / kBlock), T). Every load is issued
// before the first use (KM >= k pairs at clamped indices; the extra ones are not summed),
// then the sum runs in pair order.
template <int KM>
__global__ void __launch_bounds__(kBlock) combine_kernel(ExpertArgs a) {
  const int t = blockIdx.y, r = blockIdx.x * kBlock + threadIdx.x;
  if (r >= a.H) return;
  float wv[KM], ov[KM];
#pragma unroll
  for (int j = 0; j < KM; ++j) {
    const int p = t * a.k + min(j, a.k - 1);
    wv[j] = a.topk_w[p];
    ov[j] = a.o[(int64_t)p * a.H + r];
  }
  const float osh = a.has_shared ? a.o[(int64_t)(a.T * a.k + t) * a.H + r] : 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < KM; ++j)
    if (j < a.k) s = fmaf(wv[j], ov[j], s);
  if (a.has_shared) s += osh;
  if (a.resid) s += bf16_to_f32(a.resid[(int64_t)t * a.H + r]);   // the residual add
  a.y[(int64_t)t * a.H + r] = (uint16_t)f32_to_bf16_rne(s);
}

hipError_t launch_hquant(const ExpertArgs& a, hipStream_t s) {
  return launch_kernel(K_HQUANT, hquant_kernel, dim3(a.T * a.k), dim3(kBlock), 0, s, a);
}

hipError_t launch_combine(const ExpertArgs& a, hipStream_t s) {
  const dim3 grid((a.H + kBlock - 1) / kBlock, a.T);
  if (a.k <= 2) return launch_kernel(K_COMBINE, combine_kernel<2>, grid, dim3(kBlock), 0, s, a);
  if (a.k <= 4) return launch_kernel(K_COMBINE, combine_kernel<4>, grid, dim3(kBlock), 0, s, a);
  if (a.k <= 8) return launch_kernel(K_COMBINE, combine_kernel<8>, grid, dim3(kBlock), 0, s, a);
  return launch_kernel(K_COMBINE, combine_kernel<16>, grid, dim3(kBlock), 0, s, a);
}

}  // namespace moe
