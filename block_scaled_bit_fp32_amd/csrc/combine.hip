// Kernels between and after the expert GEMVs:
//   hquant_kernel   re-quantizes each routed pair's SwiGLU output h (FP32, one row of I)
//                   per the layer's activation format (Four-Over-Six NVFP4 or FP8 per
//                   row) -- the quantize-before-down step of the Inkling page's MoE with
//                   fused activation quantization, done once per pair.
//   combine_kernel  y[t][r] = sum_j w[t][j] * o[t*k+j][r] (+ o_shared[t][r]), FP32 in that
//                   order, rounded to BF16 -- the weighted combine.
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
  } else {
    quant_row_fp8(row, a.I, a.hq_codes + (int64_t)p * a.I, a.hq_scale + p, red);
    if (a.dbg_codes) quant_row_fp8(row, a.I, a.dbg_codes + (int64_t)p * a.I, a.dbg_scale + p, red);
  }
}

__global__ void __launch_bounds__(kBlock) combine_kernel(ExpertArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (idx >= (int64_t)a.T * a.H) return;
  const int t = (int)(idx / a.H), r = (int)(idx % a.H);
  float s = 0.0f;
  for (int j = 0; j < a.k; ++j) {
    const int p = t * a.k + j;
    s = fmaf(a.topk_w[p], a.o[(int64_t)p * a.H + r], s);
  }
  if (a.has_shared) s += a.o[(int64_t)(a.T * a.k + t) * a.H + r];
  a.y[idx] = (uint16_t)f32_to_bf16_rne(s);
}

hipError_t launch_hquant(const ExpertArgs& a, hipStream_t s) {
  return launch_kernel(K_HQUANT, hquant_kernel, dim3(a.T * a.k), dim3(kBlock), 0, s, a);
}

hipError_t launch_combine(const ExpertArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.T * a.H;
  return launch_kernel(K_COMBINE, combine_kernel, dim3((unsigned)((n + kBlock - 1) / kBlock)), dim3(kBlock),
                       0, s, a);
}

}  // namespace moe
