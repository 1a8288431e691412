// Router GEMV + sigmoid top-k, token quantization, the standalone Four-Over-Six
// quantizer and the workspace fill kernel.
//
// route_kernel: workgroups tile (tokens x experts); each of the 4 waves reduces a quarter
// of H. The last workgroup to finish a token tile (device-scope counter after a release
// fence) selects that tile's top-k; nothing waits on another workgroup. Extra
// workgroups quantize the tokens in the same launch when the layer quantizes x.
#include <algorithm>

#include "launch.hpp"
#include "rows.hpp"

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

// ======================================================================== route
template <int ET, int TT>
__global__ void __launch_bounds__(kBlock) route_kernel(RouteArgs a) {
  __shared__ float red[(kBlock / kWave) * ET * TT];
  __shared__ int last;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int n_router = a.n_tt * a.n_et;
  if ((int)blockIdx.x >= n_router) {  // token quantization workgroups
    const int t = blockIdx.x - n_router;
    const Bf16Row row{a.x + (int64_t)t * a.H};
    if (a.afmt == A_NVFP4_4O6) {
      quant_row_nvfp4(row, a.H, a.xq_codes + (int64_t)t * (a.H / 2),
                      a.xq_scales + (int64_t)t * (a.H / 16), a.xq_scale + t, nullptr, red);
    } else {
      quant_row_fp8(row, a.H, a.xq_codes + (int64_t)t * a.H, a.xq_scale + t, red);
    }
    return;
  }
  const int tt = blockIdx.x / a.n_et, et = blockIdx.x % a.n_et;
  const int t0 = tt * TT, e0 = et * ET;
  const int nt = min(TT, a.T - t0), ne = min(ET, a.E - e0);
  const int quarter = a.H / 4;        // elements of K per wave
  const int kb = wave * quarter;
  float acc[ET][TT];
#pragma unroll
  for (int e = 0; e < ET; ++e)
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[e][t] = 0.0f;
  for (int c = lane * 4; c < quarter; c += kWave * 4) {
    const int h = kb + c;
    float4 wv[ET];
#pragma unroll
    for (int e = 0; e < ET; ++e)
      wv[e] = e < ne ? *reinterpret_cast<const float4*>(a.wr + (int64_t)(e0 + e) * a.H + h)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t < nt) {
        const uint2 xb = *reinterpret_cast<const uint2*>(a.x + (int64_t)(t0 + t) * a.H + h);
        const float x0 = bf16_to_f32(xb.x & 0xFFFFu), x1 = bf16_to_f32(xb.x >> 16);
        const float x2 = bf16_to_f32(xb.y & 0xFFFFu), x3 = bf16_to_f32(xb.y >> 16);
#pragma unroll
        for (int e = 0; e < ET; ++e)
          acc[e][t] = fmaf(wv[e].w, x3, fmaf(wv[e].z, x2, fmaf(wv[e].y, x1, fmaf(wv[e].x, x0, acc[e][t]))));
      }
    }
  }
#pragma unroll
  for (int e = 0; e < ET; ++e)
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float v = group_sum<kWave>(acc[e][t]);
      if (lane == 0) red[(wave * ET + e) * TT + t] = v;
    }
  __syncthreads();
  if ((int)threadIdx.x < ET * TT) {
    const int e = threadIdx.x / TT, t = threadIdx.x % TT;
    if (e < ne && t < nt) {
      float v = red[(0 * ET + e) * TT + t];
#pragma unroll
      for (int w = 1; w < kBlock / kWave; ++w) v += red[(w * ET + e) * TT + t];
      if (a.bias) v += a.bias[e0 + e];
      store_coherent(a.logits + (int64_t)(t0 + t) * a.E + e0 + e, v);
    }
  }
  if (!arrive_last(&a.counters[tt], (uint32_t)a.n_et, &last)) return;
  // ---- top-k for the tile's tokens: one wave per token, k rounds of a wave argmax
  for (int ti = wave; ti < nt; ti += kBlock / kWave) {
    const int t = t0 + ti;
    const float* lg = a.logits + (int64_t)t * a.E;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = lane + kWave * i;
      v[i] = e < a.E ? load_coherent(lg + e) : -INFINITY;
    }
    uint32_t taken = 0;
    float myv = 0.0f;
    int mye = 0;
    for (int j = 0; j < a.k; ++j) {
      float bv = -INFINITY;
      int be = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = lane + kWave * i;
        if (e < a.E && !((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
          bv = v[i];
          be = e;
        }
      }
#pragma unroll
      for (int o = kWave / 2; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (ov > bv || (ov == bv && oe < be)) {
          bv = ov;
          be = oe;
        }
      }
      if ((be & (kWave - 1)) == lane) taken |= 1u << (be / kWave);
      if (lane == j) {
        myv = bv;
        mye = be;
      }
    }
    const float s = lane < a.k ? 1.0f / (1.0f + expf(-myv)) : 0.0f;
    float tot = 0.0f;
    for (int j = 0; j < a.k; ++j) tot += __shfl(s, j, kWave);
    if (lane < a.k) {
      a.ids[(int64_t)t * a.k + lane] = mye;
      a.w[(int64_t)t * a.k + lane] = s / tot;
    }
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

hipError_t launch_route(const RouteArgs& a, int n_quant, hipStream_t s) {
  const int grid = a.n_tt * a.n_et + n_quant;
  if (a.ET == 1) return launch_kernel(K_ROUTE, route_kernel<1, 8>, dim3(grid), dim3(kBlock), 0, s, a);
  return launch_kernel(K_ROUTE, route_kernel<4, 8>, dim3(grid), dim3(kBlock), 0, s, a);
}

}  // namespace moe
