// Sigmoid / softmax top-k of one token by one wave, shared by the top-k kernel and the
// gate/up kernel's fused routing (both take the same steps, so they select the same
// experts and compute the same weights bit for bit).
#pragma once
#include <utility>

#include "device.hpp"

namespace moe {

// The k largest of lg[0..E), largest first, ties to the lower expert index; weights are
// the sigmoids (softmax = 0) or the exponentials (softmax = 1) of the selected values,
// renormalized over the selection (FP32). The values are the selected entries of lg, or,
// when raw is given (a router bias that only selects: lg holds logit + bias, raw the bare
// logits), the selected entries of raw.
//
// Layout: expert e sits in lane e / NK, slot e % NK (E <= 64 * NK), so lane order is
// expert order. Keys are the logits' order-preserving bits (0 marks an empty slot, a
// valid key is at least 1). Each lane first sorts its NK (key, slot) pairs, largest key
// first and the lower slot first among equal keys (a sorting network on 64-bit (key,
// ~slot) composites). A round then takes the wave maximum m of the lanes' heads (DPP),
// picks the lowest lane whose head equals m (its head is then the lowest expert index
// holding m, since lanes and slots are both in expert order) and pops that lane's list.
// k rounds select the k experts in order. A wave instruction costs the same whether the
// lanes need it or not, so the rounds are kept short: one fused DPP maximum per level,
// a ballot and a find-first for the winner, a register shift for the pop.
// Lane j < k returns the j-th expert and its weight. Whole-wave call (uniform arguments).
//
// The loads (one logit, and with RAW one bare logit, per slot) and the selection are
// separate steps, so that a caller can issue the loads early.
template <int NK, bool RAW>
struct TopkIn {
  float v[NK];
  float r[RAW ? NK : 1];
};

template <int NK, bool RAW>
__device__ __forceinline__ void wave_topk_load(const float* lg, const float* raw, int E, TopkIn<NK, RAW>& in) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int e = min(NK * lane + i, E - 1);
    in.v[i] = lg[e];
    if constexpr (RAW) in.r[i] = raw[e];
  }
}

// Comparator lists that sort NK values with the larger one first: optimal networks for
// 2, 4, 6 and 8 inputs, Batcher's bitonic network for 16.
template <int NK>
struct SortNet;
template <>
struct SortNet<1> {
  static constexpr int n = 0;
  static constexpr int8_t ab[1][2] = {{0, 0}};
};
template <>
struct SortNet<2> {
  static constexpr int n = 1;
  static constexpr int8_t ab[1][2] = {{0, 1}};
};
template <>
struct SortNet<4> {
  static constexpr int n = 5;
  static constexpr int8_t ab[5][2] = {{0, 1}, {2, 3}, {0, 2}, {1, 3}, {1, 2}};
};
template <>
struct SortNet<6> {
  static constexpr int n = 12;
  static constexpr int8_t ab[12][2] = {{0, 5}, {1, 3}, {2, 4}, {1, 2}, {3, 4}, {0, 3},
                                       {2, 5}, {0, 1}, {2, 3}, {4, 5}, {1, 2}, {3, 4}};
};
template <>
struct SortNet<8> {
  static constexpr int n = 19;
  static constexpr int8_t ab[19][2] = {{0, 1}, {2, 3}, {4, 5}, {6, 7}, {0, 2}, {1, 3}, {4, 6},
                                       {5, 7}, {1, 2}, {5, 6}, {0, 4}, {1, 5}, {2, 6}, {3, 7},
                                       {2, 4}, {3, 5}, {1, 2}, {3, 4}, {5, 6}};
};
template <>
struct SortNet<16> {
  static constexpr int n = 80;
  // bitonic: blocks of size 2, 4, 8, 16; a block's direction alternates with bit `size`
  static constexpr int8_t ab[80][2] = {
      {0, 1},  {3, 2},   {4, 5},   {7, 6},   {8, 9},   {11, 10}, {12, 13}, {15, 14},   // size 2
      {0, 2},  {1, 3},   {6, 4},   {7, 5},   {8, 10},  {9, 11},  {14, 12}, {15, 13},   // size 4
      {0, 1},  {2, 3},   {5, 4},   {7, 6},   {8, 9},   {10, 11}, {13, 12}, {15, 14},
      {0, 4},  {1, 5},   {2, 6},   {3, 7},   {12, 8},  {13, 9},  {14, 10}, {15, 11},   // size 8
      {0, 2},  {1, 3},   {4, 6},   {5, 7},   {10, 8},  {11, 9},  {14, 12}, {15, 13},
      {0, 1},  {2, 3},   {4, 5},   {6, 7},   {9, 8},   {11, 10}, {13, 12}, {15, 14},
      {0, 8},  {1, 9},   {2, 10},  {3, 11},  {4, 12},  {5, 13},  {6, 14},  {7, 15},    // size 16
      {0, 4},  {1, 5},   {2, 6},   {3, 7},   {8, 12},  {9, 13},  {10, 14}, {11, 15},
      {0, 2},  {1, 3},   {4, 6},   {5, 7},   {8, 10},  {9, 11},  {12, 14}, {13, 15},
      {0, 1},  {2, 3},   {4, 5},   {6, 7},   {8, 9},   {10, 11}, {12, 13}, {14, 15}};
};

// Wave maximum of a 32-bit value, as a scalar: four DPP levels within each row of 16
// lanes, then row_bcast:15 and row_bcast:31 carry the row maxima up to lane 63.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, false);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v) {
  v = dpp_max_step<0xB1, 0xF>(v);    // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E, 0xF>(v);    // quad_perm [2,3,0,1]
  v = dpp_max_step<0x124, 0xF>(v);   // row_ror:4
  v = dpp_max_step<0x128, 0xF>(v);   // row_ror:8
  v = dpp_max_step<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
// Sum (or maximum) of lanes 0..15, as a scalar: xor 1 and xor 2 within quads, then the
// rotations by 4 and 8; lane 0's value is ((q0 + q1) + (q2 + q3)) over the quad values q.
template <bool MAX>
__device__ __forceinline__ float row0_reduce(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false)));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
}

// The lists live in vector registers typed as vectors, so that every access has a constant
// index and the pop is one vector select (an array here can be turned into an indexed
// stack object by the optimizer, which costs a compare chain per element).
template <int NK>
using U64v = uint64_t __attribute__((ext_vector_type(NK)));
template <int NK>
using F32v = float __attribute__((ext_vector_type(NK)));
template <class V, size_t... I>
__device__ __forceinline__ V shift_down(V c, std::index_sequence<I...>) {
  return __builtin_shufflevector(c, V{}, (int)(I + 1)...);   // c[1..NK) then one zero
}

template <int NK, bool RAW>
__device__ __forceinline__ void wave_topk_select(const TopkIn<NK, RAW>& in, int E, int k, bool softmax, int& mye,
                                                 float& myw) {
  const int lane = threadIdx.x & (kWave - 1);
  U64v<NK> c;   // (key << 32) | ~slot
  F32v<NK> rv;
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const uint32_t o = float_order_key(in.v[i]);
    const uint32_t key = NK * lane + i < E ? (o > 1u ? o : 1u) : 0u;
    c[i] = ((uint64_t)key << 32) | (uint32_t)~(uint32_t)i;
    rv[i] = RAW ? in.r[RAW ? i : 0] : 0.0f;
  }
#pragma unroll
  for (int q = 0; q < SortNet<NK>::n; ++q) {
    const int a = SortNet<NK>::ab[q][0], b = SortNet<NK>::ab[q][1];
    const bool sw = c[b] > c[a];
    const uint64_t ca = c[a], cb = c[b];
    c[a] = sw ? cb : ca;
    c[b] = sw ? ca : cb;
    if constexpr (RAW) {
      const float ra = rv[a], rb = rv[b];
      rv[a] = sw ? rb : ra;
      rv[b] = sw ? ra : rb;
    }
  }
  float myv = 0.0f;
  mye = 0;
  for (int j = 0; j < k; ++j) {
    const uint64_t h = c[0];
    const uint32_t head = (uint32_t)(h >> 32);
    const uint32_t m = wave_max_dpp(head);
    const int wl = __ffsll((long long)__ballot(head == m)) - 1;   // the lowest lane holding m
    const int slot = (int)~(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)h, wl);
    const float bv = RAW ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int((float)rv[0]), wl))
                         : float_from_order_key(m);
    const bool me = lane == wl;
    c = me ? shift_down(c, std::make_index_sequence<NK>{}) : c;
    if constexpr (RAW) rv = me ? shift_down(rv, std::make_index_sequence<NK>{}) : rv;
    if (lane == j) {
      mye = NK * wl + slot;
      myv = bv;
    }
  }
  float s;
  if (softmax) {   // exp(v - max v): with a selection bias the largest value need not come first
    const float mx = RAW ? row0_reduce<true>(lane < k ? myv : -INFINITY)
                         : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(myv), 0));
    s = lane < k ? expf(myv - mx) : 0.0f;
  } else {
    s = lane < k ? 1.0f / (1.0f + expf(-myv)) : 0.0f;
  }
  const float tot = row0_reduce<false>(s);   // k <= 16: the selection sits in lanes 0..15
  myw = lane < k ? s / tot : 0.0f;
}

template <int NK>
__device__ __forceinline__ void wave_topk(const float* lg, int E, int k, const float* raw, bool softmax, int& mye,
                                          float& myw) {
  if (raw) {
    TopkIn<NK, true> in;
    wave_topk_load<NK, true>(lg, raw, E, in);
    wave_topk_select<NK, true>(in, E, k, softmax, mye, myw);
  } else {
    TopkIn<NK, false> in;
    wave_topk_load<NK, false>(lg, nullptr, E, in);
    wave_topk_select<NK, false>(in, E, k, softmax, mye, myw);
  }
}

// Routing fused into another kernel's prologue calls wave_topk_load and wave_topk_select
// itself, built per slot count (fused_topk_slots(E) of plan.hpp) and per presence of bare
// logits: it takes the same steps as the top-k kernel for that kind of layer, so both
// select the same experts and compute the same weights bit for bit.

}  // namespace moe
