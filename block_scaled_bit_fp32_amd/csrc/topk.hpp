// Sigmoid top-k of one token by one wave, shared by the top-k kernel and the gate/up
// kernel's fused routing (both take the same steps, so they select the same experts and
// compute the same weights bit for bit).
#pragma once
#include "device.hpp"

namespace moe {

// The k largest of lg[0..E), largest first, ties to the lower expert index; weights are
// the sigmoids (softmax = 0) or the exponentials (softmax = 1) of the selected values,
// renormalized over the selection in selection order (FP32). The values are the
// selected entries of lg, or, when raw is given (a router bias that only selects: lg
// holds logit + bias, raw the bare logits), the selected entries of raw. Expert e
// sits in lane e % 64, slot e / 64 (E <= 64 * NK); keys are the logits' order-preserving
// bits (0 marks an empty or taken slot; a valid key is at least 1). Each lane keeps its
// best slot (the lowest slot among equal keys, i.e. the lowest index); a round takes the
// wave maximum of those, the lane holding it (the lowest index if several do), and only
// that lane rescans its slots. Lane j < k returns the j-th expert and its weight.
// Whole-wave call (uniform arguments).
// The loads (one logit per slot) and the selection are separate steps, so that a caller
// can issue the loads early: wave_topk_load then wave_topk_select (wave_topk does both).
template <int NK>
__device__ __forceinline__ void wave_topk_load(const float* lg, int E, float (&lv)[NK]) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int i = 0; i < NK; ++i) lv[i] = lg[min(lane + kWave * i, E - 1)];
}
// RAW: the weights take raw[] (a load per selected expert). A compile-time choice: a
// load behind a run-time branch would make the wait for its value drain every load the
// caller has in flight.
template <int NK, bool RAW>
__device__ __forceinline__ void wave_topk_select(const float (&lv)[NK], int E, int k, const float* raw, bool softmax,
                                                 int& mye, float& myw) {
  const int lane = threadIdx.x & (kWave - 1);
  uint32_t key[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = lane + kWave * i;
    const uint32_t o = float_order_key(lv[i]);
    key[i] = e < E ? (o > 1u ? o : 1u) : 0u;
  }
  uint32_t lb = 0;
  int li = 0;
  auto rescan = [&]() {
    lb = key[0];
    li = 0;
#pragma unroll
    for (int i = 1; i < NK; ++i)
      if (key[i] > lb) { lb = key[i]; li = i; }
  };
  rescan();
  float myv = 0.0f;
  mye = 0;
  for (int j = 0; j < k; ++j) {
    const uint32_t m = wave_ext_u32<true>(lb);
    const uint64_t tied = __ballot(lb == m);
    int be;
    if (__popcll(tied) == 1) {
      const int wl = __ffsll((long long)tied) - 1;
      be = wl + kWave * __builtin_amdgcn_readlane(li, wl);
    } else {   // equal keys in several lanes: the lowest index among them
      be = (int)wave_ext_u32<false>(lb == m ? (uint32_t)(lane + kWave * li) : 0xFFFFFFFFu);
    }
    if (lane == (be & (kWave - 1))) {
      const int taken = be / kWave;
#pragma unroll
      for (int i = 0; i < NK; ++i)
        if (i == taken) key[i] = 0u;
      rescan();
    }
    if (lane == j) {
      myv = float_from_order_key(m);
      mye = be;
    }
  }
  if constexpr (RAW) myv = raw[lane < k ? mye : 0];   // one load per selected expert
  float s;
  if (softmax) {   // exp(v - max v): with a selection bias the largest value need not come first
    float mx = -INFINITY;
    for (int j = 0; j < k; ++j) mx = fmaxf(mx, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myv), j)));
    s = lane < k ? expf(myv - mx) : 0.0f;
  } else {
    s = lane < k ? 1.0f / (1.0f + expf(-myv)) : 0.0f;
  }
  float tot = 0.0f;
  for (int j = 0; j < k; ++j) tot += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s), j));
  myw = lane < k ? s / tot : 0.0f;
}
template <int NK>
__device__ __forceinline__ void wave_topk(const float* lg, int E, int k, const float* raw, bool softmax, int& mye,
                                          float& myw) {
  float lv[NK];
  wave_topk_load<NK>(lg, E, lv);
  if (raw)
    wave_topk_select<NK, true>(lv, E, k, raw, softmax, mye, myw);
  else
    wave_topk_select<NK, false>(lv, E, k, nullptr, softmax, mye, myw);
}

}  // namespace moe
