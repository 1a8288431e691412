// Host/device shared plain structs: launch plans and kernel arguments.
#pragma once
#include <stdint.h>

namespace moe {

enum WFmt : int { W_BF16 = 0, W_NVFP4 = 1, W_MXFP4 = 2, W_MXFP8 = 3 };
enum AFmt : int { A_BF16 = 0, A_NVFP4_4O6 = 1, A_FP8_TOKEN = 2, A_MXFP4 = 3, A_MXFP8 = 4 };

// Activation formats with one FP32 scale per row (the rest carry E8M0 scales per 32).
inline constexpr bool afmt_row_scaled(int af) { return af == A_NVFP4_4O6 || af == A_FP8_TOKEN; }

// Elements one lane reads per 16-byte weight load.
inline constexpr int elems_per_piece(int fmt) {
  return fmt == W_BF16 ? 8 : (fmt == W_MXFP8 ? 16 : 32);
}

// How a workgroup (4 waves) walks the rows of one weight class (routed or shared).
//   LPR lanes share a row (power of two); G = 64 / LPR rows per wave at a time; each
//   lane holds RPL rows (gate/up: RPL = 2, the gate row and the up row of the same
//   intermediate index, so SwiGLU happens in registers; down: RPL = 1). A row-step covers
//   RS = 4 * G * RPL rows. Lane jl of a row reads the 16-byte pieces at element
//   offsets (s * LPR + jl) * EPL, s < NP = K / (LPR * EPL), in NB batches of NPB.
//   A work unit is one expert with a group of at most NG of its tokens, whose
//   activations (full K, esize bytes per element) sit in LDS while the unit streams.
//   A step of a unit with n tokens costs cw + ct * n (workgroups split the summed
//   cost evenly).
struct GemvMap {
  int LPR, G, RPL, RS, NP, NPB, NB, NG, esize, cw, ct;
  // launch constants the host works out, so that kernel prologues divide nothing:
  int lg;          // log2(LPR)
  int steps;       // row-steps per unit
  float inv_steps; // 1 / steps
  int cap;         // rows of the class the LDS tile holds (at most kWinRows)
  int win;         // rows the first window may hold (prologue register slots)
};

constexpr int kWinRows = 64;   // most token rows one staged window of units holds
// GEMV walks with NVFP4 weights: LDS per wave for a batch's block scales (after the
// activation tile; RPL x G rows x NPB x LPR x 2 bytes <= 1 KB)
constexpr int kScaleStageWave = 1024;
constexpr int kScaleStageBytes = 4 * kScaleStageWave;
constexpr int kPairMax = 64;   // GEMV kernels: one unit per (token, expert) pair up to this many pairs
constexpr int kFusedTopkSlots = 8;          // routing fused into gate/up: E <= 64 * this
// Slots per lane of the routing fused into the gate/up GEMV (a kernel per count): E <= 128
// in 2, E <= 256 in 4, E <= 512 in 8.
inline constexpr int fused_topk_slots(int E) { return E <= 128 ? 2 : (E <= 256 ? 4 : 8); }
constexpr int kTokParkBytes = 8 * 256 * 16;   // activation bytes the token walk's prologue holds in registers
constexpr int kTokJMax = 8;     // token mode of the down GEMV: experts per token (k + shared)
constexpr int kTokPieces = 3;   // and pieces per lane of a row-step (NP, one batch)

// Routed class table capacity: one entry per selected expert, or per pair in pair mode.
inline constexpr int routed_capacity(int E, int P) { return P <= kPairMax ? P : (E < P ? E : P); }
// Bytes of the expert kernels' LDS before the activation tile: token masks (ceil(T/64)
// words per expert), first pairs and row bases per expert, ids, span, the routed and
// shared class tables, the staged rows' scales and the global weight scales of every
// expert. Am = routed class capacity, P = T*k class rows.
inline int expert_lds_list_bytes(int E, int T, int k) {
  const int P = T * k, Am = routed_capacity(E, P), nw = (T + 63) / 64;
  return (E * 8 * nw + E * 8 + P * 4 + 16 + 32 + 4 * (5 * Am + 3) + 12 * P + 4 * (5 + 3) + 12 * T +
          3 * kWinRows * 4 + 4 * (2 * E + 2) + 15) / 16 * 16;
}

// Grouped (MFMA) expert kernels, one weight class: each wave owns 32 weight rows of a
// row tile (gate/up: 16 gate rows and the 16 matching up rows; down: 32 hidden rows),
// a unit is an expert with up to NG = 32 of its tokens, and the K dimension is walked in
// stages of KS elements (each lane holds 64 bytes of weights per stage: FP4 256, FP8
// 128, BF16 64 elements per stage). Activations of a stage sit in LDS as BF16 (or as
// raw MX codes with their scales on the scaled MFMA).
// K elements per stage of the grouped kernels: 64 bytes of weights per lane, both
// halves of the wave.
inline constexpr int group_ks(int fmt) { return fmt == W_BF16 ? 64 : (fmt == W_MXFP8 ? 128 : 256); }
// Grouped kernels: each stage's weights (4 waves x 32 rows x 128 bytes) pass through LDS
// after the activation buffers. One buffer: a wave reads only its own rows, and it writes
// the next stage's rows after its reads of the current stage's (LDS operations of one
// wave complete in order).
constexpr int kGWeightStage = 4 * 32 * 128;
constexpr int kGWeightLds = kGWeightStage;
// LDS of a grouped launch that keeps two workgroups on a compute unit (160 KB on gfx950)
constexpr int kGroupedLdsMax = 80 * 1024;

struct GroupMap {
  int KS, NS;        // K elements per stage, stages per row tile
  int steps;         // row tiles per expert
  int NG;            // tokens per unit
  int cw, ct;        // cost of one stage of a row tile: cw + ct * tokens
  int tstride;       // LDS bytes per staged token row (padded)
  int scaled;        // MX weights on the scaled MFMA: raw activation codes staged, then
                     // 8 E8M0 bytes per token
};

struct WTensor {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* gscale;
  int64_t code_row_bytes;
  int64_t scale_row_bytes;
  int rows;   // rows per expert
  int K;
  int gs_per_expert;
  int fmt;
};

struct RouteArgs {
  const uint16_t* x;
  const float* wr;
  const float* bias;
  int T, H, E, k, afmt;
  int TT, ET, n_tt, n_et;   // token tile, experts per workgroup, tile counts
  float* logits;            // [T][E]
  int32_t* ids;
  float* w;
  uint8_t* xq_codes;
  uint8_t* xq_scales;
  float* xq_scale;
  int softmax;              // combine weights: softmax (1) or sigmoid (0) of the selected
  float* raw;               // [T][E] bare logits (bias for selection only: logits hold
                            // logit + bias, the weights take these), or NULL
  // RMSNorm before the layer (resid != NULL): x = RMSNorm(resid) * gamma in BF16 is the
  // layer's input; the router computes it on the fly, the per-token workgroups write it
  const uint16_t* resid;    // [T][H] residual stream, or NULL (x taken as given)
  const uint16_t* gamma;    // [H] BF16
  float eps;
  uint16_t* x_out;          // [T][H] the normalized tokens
};

struct ExpertArgs {
  const uint16_t* x;
  const uint8_t* xq_codes;
  const uint8_t* xq_scales;
  const float* xq_scale;
  const int32_t* ids;
  const float* topk_w;
  WTensor rw, sw;        // routed / shared weights of this stage
  GemvMap rmap, smap;
  GroupMap rgm, sgm;     // grouped kernels (batches of 32 tokens and up)
  int grouped;           // run the grouped kernels
  int pair_mode;         // GEMV kernels: one unit per (token, expert) pair
  int token_mode;        // down GEMV: items (token, row-step) over all of a token's
                         // experts, writing y (no combine launch); 1: an item is RS rows,
                         // 2 (wide): G rows, the waves splitting the token's experts
  int tok_items;         // token mode: items per token (H / rows per item)
  float tok_inv;         // 1 / tok_items
  float inv_k;           // 1 / k
  // pair and token modes, positions of one cost: the class's first n1 workgroups (those
  // dispatched in the first round) take q1 or q1 + 1 (the first r1 of them q1 + 1), the
  // others q2 or q2 + 1
  int pn1, pq1, pr1, pq2, pr2;
  int fuse_topk;         // gate/up GEMV in pair mode: routing from logits in the prologue,
  const float* logits;   // writing ids_out / w_out (the buffers ids / topk_w point at)
  int32_t* ids_out;
  float* w_out;
  const float* raw;      // bare logits [T][E] (bias for selection only) or NULL
  int softmax;           // softmax (1) or sigmoid (0) combine weights
  int T, H, I, Ish, E, k, has_shared, afmt;
  int max_slots;         // routed expert slots launched: min(E, T * k)
  int sh_wgs;            // workgroups of the launch that walk the shared expert
  int ncu, late16;       // compute units; weight (in 16ths) of a block dispatched after
                         // the first ncu, against 16 for the first ones
  float* h;              // [T*k + T][hs]
  int hs;
  uint8_t* hq_codes;     // [T*k][I/2 | I]
  uint8_t* hq_scales;    // [T*k][I/16]
  float* hq_scale;       // [T*k]
  float* o;              // [T*k + T][H]
  uint16_t* y;
  float* dbg_h;
  uint8_t* dbg_codes;
  uint8_t* dbg_scales;
  float* dbg_scale;
  int lds_list_bytes;    // offset of the activation tile in dynamic LDS
  int lds_act_bytes;     // size of the activation tile
  const uint16_t* resid; // [T][H] residual stream added to y before its rounding, or NULL
};

}  // namespace moe
