// C ABI of libmoe_mi355x.so: argument checks, launch planning, workspace layout and
// dispatch to the gfx950 kernels. Declarations and contracts: include/moe.h.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "plan.hpp"

namespace moe {
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_requant_mxfp4(const uint16_t* x, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                                hipStream_t s);
hipError_t launch_requant_nvfp4(const uint16_t* x, int ntensors, int64_t n, uint8_t* codes, uint8_t* scales,
                                float* gscale, hipStream_t s);
hipError_t launch_requant_fp8b_mxfp4(const uint8_t* w, const float* bscale, int64_t rows, int cols, int block_rows,
                                     int block_cols, uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_requant_mxfp8(const uint16_t* x, int64_t nblocks, uint8_t* codes, uint8_t* scales,
                                hipStream_t s);
hipError_t launch_quantize_nvfp4(const uint16_t* x, int rows, int cols, uint8_t* codes,
                                 uint8_t* scales, float* g, uint8_t* choice, hipStream_t s);
hipError_t launch_route(const RouteArgs& a, int n_quant, bool topk, hipStream_t s);
#define MOE_DECL_EXPERTS(NAME)                                                              \
  hipError_t NAME(const ExpertArgs& gu, int gu_grid, size_t gu_lds, const ExpertArgs& dn,  \
                  int dn_grid, size_t dn_lds, int sf, hipStream_t s);
MOE_DECL_EXPERTS(launch_experts_bf16)
MOE_DECL_EXPERTS(launch_experts_nvfp4)
MOE_DECL_EXPERTS(launch_experts_mxfp4)
MOE_DECL_EXPERTS(launch_experts_mxfp8)
#undef MOE_DECL_EXPERTS

// Both expert kernels for the layer's (routed, shared) weight formats.
static hipError_t launch_experts(const ExpertArgs& gu, int gu_grid, size_t gu_lds,
                                 const ExpertArgs& dn, int dn_grid, size_t dn_lds, hipStream_t s) {
  const int sf = gu.has_shared ? gu.sw.fmt : gu.rw.fmt;
  switch (gu.rw.fmt) {
    case W_BF16: return launch_experts_bf16(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, sf, s);
    case W_NVFP4: return launch_experts_nvfp4(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, sf, s);
    case W_MXFP4: return launch_experts_mxfp4(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, sf, s);
    case W_MXFP8: return launch_experts_mxfp8(gu, gu_grid, gu_lds, dn, dn_grid, dn_lds, sf, s);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace moe

using namespace moe;

namespace {

thread_local std::string g_err;

constexpr int kMaxTokens = 256;    // tokens per call
constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;
constexpr int kRouteTT = 8;         // router GEMV: tokens per workgroup past kRouteSmallT tokens
constexpr int kRouteSmallT = 16;    // up to here one token per workgroup
constexpr int kLdsActBudget = 48 * 1024;   // activation tile per workgroup
constexpr size_t kAlign = 256;

moe_status_t set_err(moe_status_t st, const std::string& msg) {
  g_err = msg;
  return st;
}

size_t align_up(size_t v, size_t a = kAlign) { return (v + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool valid_wfmt(int f) { return f >= MOE_W_BF16 && f <= MOE_W_MXFP8; }

// weight bytes per row of K elements
int64_t code_row_bytes(int fmt, int K) {
  return fmt == W_BF16 ? 2 * (int64_t)K : (fmt == W_MXFP8 ? (int64_t)K : (int64_t)K / 2);
}
int64_t scale_row_bytes(int fmt, int K) {
  return fmt == W_NVFP4 ? K / 16 : (fmt == W_BF16 ? 0 : K / 32);
}

// Row mapping of one weight class (see GemvMap) for rows of length K, activations of
// `esize` bytes per element, up to ntok tokens per expert; paired = gate/up; pref = the
// pieces per lane to aim for (8, or 3 for the down rows of token-mode items).
bool plan_class(int fmt, int K, int ntok, int esize, bool paired, GemvMap& m, int pref = 8) {
  const int EPL = elems_per_piece(fmt);
  if (K <= 0 || K % EPL) return false;
  const int units = K / EPL;
  // lanes per row: the largest power of two giving every lane >= pref pieces of the row
  // (fewer lanes per row put more rows on a wave, so each activation piece read from LDS
  // serves more rows, and the row-sum takes one shuffle step less), else >= 3. Pieces per
  // batch: the largest divisor of NP up to 4. A mapping whose NVFP4 block scales could not
  // be staged (several batches of a row with a batch's scales not a multiple of 16 bytes)
  // falls back to >= 3.
  int LPR = 1, NP = units, NPB = 1;
  for (int min_pieces : {pref, 3}) {
    LPR = 1;
    for (int l = 64; l >= 1; l >>= 1)
      if (units % l == 0 && units / l >= min_pieces) { LPR = l; break; }
    NP = units / LPR;
    NPB = 1;
    for (int d = 4; d >= 1; --d)
      if (NP % d == 0) { NPB = d; break; }
    if (fmt != W_NVFP4 || NP == NPB || (NPB * LPR * 2) % 16 == 0) break;
  }
  m.LPR = LPR;
  m.G = 64 / LPR;
  m.NP = NP;
  m.NPB = NPB;
  m.NB = NP / NPB;
  m.RPL = paired ? 2 : 1;
  m.RS = 4 * m.G * m.RPL;
  // tokens per LDS pass: 1, 2 or 4 (a group of 3 runs the 4-token code, which reads and
  // discards a 4th slot, so groups are powers of two); FP32 tiles 2 at most
  int NG = ntok <= 1 ? 1 : (ntok == 2 || esize == 4 ? 2 : 4);
  while (NG > 1 && NG * K * esize > kLdsActBudget) NG /= 2;
  if (NG * K * esize > kLdsActBudget) return false;
  m.NG = NG;
  m.esize = esize;
  return true;
}

struct Plan {
  GemvMap gu_r, gu_s, dn_r, dn_s;
  int max_slots;
  size_t gu_lds, dn_lds, list_bytes, gu_tile, dn_tile;
  bool grouped;                       // batches of kGroupedMinT tokens and up
  bool token;                         // the down GEMV can run in token mode
  GroupMap gu_rg, gu_sg, dn_rg, dn_sg;
};

constexpr int kGroupedMinT = 32;      // the grouped (MFMA) kernels from this batch on (4-bit weights)
constexpr int kGroupedMinTSharedBf16 = 8;   // ... with a BF16 shared expert
constexpr int kGroupedMinTWide = 24;        // ... with BF16 or MXFP8 routed weights
constexpr int kTokPctGateup = 200;    // GEMV cost model: token-term scale (see set_costs)
constexpr int kTokPctDown = 100;
constexpr int kLateGateup16 = 13;     // GEMV kernels: weight of a second-round workgroup,
constexpr int kLateDown16 = 14;       // in 16ths (timestamps: they end ~15% / ~7% later)
constexpr int kGroupTok = 32;         // tokens per unit in the grouped kernels

// Grouped map of one weight class: rows of K elements, `rows_per_tile` rows (or
// intermediate indices for gate/up) per row tile, BF16 activations staged. False if the
// shape does not tile.
// mx_bits: 4 or 8 for MX weights on the scaled MFMA with 4- or 8-bit activation codes
// (staged raw), 0 otherwise.
bool plan_group(int fmt, int K, int rows, int rows_per_tile, int mx_bits, GroupMap& g) {
  const int KS = group_ks(fmt);
  if (K % KS || rows % rows_per_tile) return false;
  g.KS = KS;
  g.NS = K / KS;
  g.steps = rows / rows_per_tile;
  g.NG = kGroupTok;
  // a row tile moves NS stages of 4 waves x 64 bytes x 64 lanes of weights (cw: 256-byte
  // units); each token adds a share of MFMA and staging work
  g.cw = g.NS * 64;
  g.ct = g.NS * 2;
  g.scaled = mx_bits ? 1 : 0;
  g.tstride = mx_bits ? KS * mx_bits / 8 + 16 : KS * 2 + 16;
  return true;
}

// LDS bytes of one staging buffer of a grouped class.
size_t group_buf_bytes(const GroupMap& g) { return (size_t)kGroupTok * g.tstride + (g.scaled ? 8 * kGroupTok : 0); }

// Weight bytes per element, times 2 (FP4 1, MXFP8 2, BF16 4; block scales ignored).
int wbytes_x2(int fmt) { return fmt == W_BF16 ? 4 : (fmt == W_MXFP8 ? 2 : 1); }

// Cost weights of one row-step (see GemvMap) over rows of K elements: weight bytes
// against activation work (a token costs half a step's weight bytes for FP4 weights and
// BF16 activations).
// tok_pct scales the token term: per-workgroup timestamps on the NVFP4 Flint layer at
// T = 8 put a 4-token BF16 gate/up step at about 2.4x a 1-token step (token term x2);
// the FP32 down steps fit the byte model (x1).
void set_costs(GemvMap& m, int fmt, int K, int tok_pct) {
  const int64_t elems = (int64_t)m.RS * K;
  m.cw = (int)std::max<int64_t>(1, elems * wbytes_x2(fmt) / 256);
  m.ct = (int)std::max<int64_t>(1, elems * m.esize * tok_pct / (1024 * 100));
}

// Row maps of both expert kernels and their LDS needs. Gate/up row-steps cover RS / 2
// intermediate indices (gate and up rows), down row-steps RS hidden rows.
bool make_plan(const moe_layer_t& L, int T, int path, Plan& p) {
  const int Ish = L.has_shared ? L.I_shared : L.I;
  const int sfmt = L.has_shared ? L.shared_wfmt : L.wfmt;
  const int nt = std::max(1, T);
  if (!plan_class(L.wfmt, L.H, nt, 2, true, p.gu_r) || !plan_class(sfmt, L.H, nt, 2, true, p.gu_s))
    return false;
  if (L.I % (p.gu_r.RS / 2) || Ish % (p.gu_s.RS / 2)) return false;
  // the down GEMV stages BF16: h stored as BF16, or decoded from its FP4 / FP8 codes.
  // Token-mode items (decided below) need 3 pieces per lane in one batch; where the
  // layer's shape rules them out, the down rows aim for 8 pieces per lane like gate/up.
  if (!plan_class(L.wfmt, L.I, nt, 2, false, p.dn_r, 3) || !plan_class(sfmt, Ish, nt, 2, false, p.dn_s, 3))
    return false;
  {
    const int J = L.k + (L.has_shared ? 1 : 0);
    const size_t lb = (size_t)expert_lds_list_bytes(L.E, nt, L.k);
    const size_t jb = (size_t)J * L.I * p.dn_r.esize, room = 64 * 1024 > lb ? 64 * 1024 - lb : 0;
    const bool tok = nt * L.k <= kPairMax && J <= kTokJMax && p.dn_r.NP == kTokPieces && p.dn_r.NB == 1 &&
                     (!L.has_shared || (sfmt == L.wfmt && Ish == L.I && L.afmt == A_BF16)) &&
                     jb <= (size_t)kTokParkBytes && jb <= room;
    if (!tok && (!plan_class(L.wfmt, L.I, nt, 2, false, p.dn_r) || !plan_class(sfmt, Ish, nt, 2, false, p.dn_s)))
      return false;
  }
  if (L.H % p.dn_r.RS || L.H % p.dn_s.RS) return false;
  set_costs(p.gu_r, L.wfmt, L.H, kTokPctGateup);
  set_costs(p.gu_s, sfmt, L.H, kTokPctGateup);
  set_costs(p.dn_r, L.wfmt, L.I, kTokPctDown);
  set_costs(p.dn_s, sfmt, Ish, kTokPctDown);
  // summed costs must fit an int: bound every unit by NG tokens
  auto bound = [&](const GemvMap& m, int steps, int units) {
    return (int64_t)units * steps * (m.cw + (int64_t)m.ct * m.NG);
  };
  const int ur = nt * L.k, us = L.has_shared ? nt : 0;
  if (bound(p.gu_r, L.I / (p.gu_r.RS / 2), ur) + bound(p.gu_s, Ish / (p.gu_s.RS / 2), us) > (1ll << 30) ||
      bound(p.dn_r, L.H / p.dn_r.RS, ur) + bound(p.dn_s, L.H / p.dn_s.RS, us) > (1ll << 30))
    return false;
  p.max_slots = std::min(L.E, nt * L.k);
  p.list_bytes = (size_t)expert_lds_list_bytes(L.E, nt, L.k);
  // activation tile: the rows of up to kWinRows tokens of a class, within 64 KB of LDS
  // per workgroup, but never less than one unit's NG rows
  auto tile = [&](const GemvMap& r, int Kr, const GemvMap& s, int Ks) {
    const size_t sr = (size_t)Kr * r.esize, ss = (size_t)Ks * s.esize;
    const size_t want = std::max(std::min<size_t>(ur, kWinRows) * sr,
                                 L.has_shared ? std::min<size_t>(us, kWinRows) * ss : 0);
    const size_t need = std::max(r.NG * sr, L.has_shared ? s.NG * ss : 0);
    const size_t room = 64 * 1024 > p.list_bytes ? 64 * 1024 - p.list_bytes : 0;
    return align_up(std::max(need, std::min(want, room)), 16);
  };
  p.gu_tile = tile(p.gu_r, L.H, p.gu_s, L.H);
  p.dn_tile = tile(p.dn_r, L.I, p.dn_s, Ish);
  // token mode of the down GEMV (pair mode; a shared expert of the routed format and
  // size taking the same FP32 h): the J activation rows of one token in the tile and in
  // the prologue's registers
  {
    const int J = L.k + (L.has_shared ? 1 : 0);
    const size_t jb = (size_t)J * L.I * p.dn_r.esize;
    const size_t room = 64 * 1024 > p.list_bytes ? 64 * 1024 - p.list_bytes : 0;
    p.token = nt * L.k <= kPairMax && J <= kTokJMax && p.dn_r.NP == kTokPieces && p.dn_r.NB == 1 &&
              (!L.has_shared || (sfmt == L.wfmt && Ish == L.I && L.afmt == A_BF16)) &&
              jb <= (size_t)kTokParkBytes && jb <= room;
    if (p.token) p.dn_tile = std::max(p.dn_tile, align_up(jb, 16));
  }
  // NVFP4 walks stage each batch's block scales in 1 KB of LDS per wave after the tile,
  // 16-byte chunks of the wave's rows: with several batches per row, a row's scales of one
  // batch (NPB x LPR x 2 bytes) must be a multiple of 16 (true for K a multiple of 256)
  const bool nv_r = L.wfmt == W_NVFP4, nv_s = sfmt == W_NVFP4;
  auto chunked = [](const GemvMap& m) { return m.NB == 1 || (m.NPB * m.LPR * 2) % 16 == 0; };
  if (nv_r && !(chunked(p.gu_r) && chunked(p.dn_r))) return false;
  if (nv_s && !(chunked(p.gu_s) && chunked(p.dn_s))) return false;
  const size_t stage = nv_r || nv_s ? (size_t)kScaleStageBytes : 0;
  p.gu_lds = p.list_bytes + p.gu_tile + stage;
  p.dn_lds = p.list_bytes + p.dn_tile + stage;
  // the kernels' launch constants (so that their prologues divide nothing): steps per
  // unit, rows the tile holds, rows the first window's register slots hold (4 slots per
  // thread for gate/up, 12 for down, 16-byte slots)
  auto consts = [&](GemvMap& m, int K, int steps, size_t tile, int slots) {
    m.lg = __builtin_ctz((unsigned)m.LPR);
    m.steps = steps;
    m.inv_steps = 1.0f / (float)steps;
    m.cap = (int)std::min<size_t>(kWinRows, tile / ((size_t)K * m.esize));
    m.win = slots * 256 / (K * m.esize / 16);
  };
  consts(p.gu_r, L.H, L.I / (p.gu_r.RS / 2), p.gu_tile, 4);
  consts(p.gu_s, L.H, Ish / (p.gu_s.RS / 2), p.gu_tile, 4);
  consts(p.dn_r, L.I, L.H / p.dn_r.RS, p.dn_tile, 12);
  consts(p.dn_s, Ish, L.H / p.dn_s.RS, p.dn_tile, 12);
  // grouped kernels: gate/up tiles of 64 intermediate indices, down tiles of 128 rows
  // automatic choice (graph-timed crossovers of both kernel pairs on the synthetic layers):
  // a BF16 shared expert is read once per 32 tokens instead of once per 4, which pays from
  // 8 tokens on (Flint BF16 T = 8: 95 against 111 us; Mistral a8w4: 182 against 236 us);
  // BF16 or MXFP8 routed weights, whose GEMV decode is the dearest, from 24 (Inkling MXFP8:
  // even at 16, grouped ahead from 32); 4-bit weights from 32 tokens when units hold many
  // tokens (a shared expert, or T*k >= E).
  const bool bf16_shared = L.has_shared && L.shared_wfmt == MOE_W_BF16;
  const bool wide_w = L.wfmt == W_BF16 || L.wfmt == W_MXFP8;
  const bool auto_grouped = bf16_shared ? T >= kGroupedMinTSharedBf16
                            : wide_w    ? T >= kGroupedMinTWide
                                        : T >= kGroupedMinT && (L.has_shared || T * L.k >= L.E);
  const bool want = path == MOE_PATH_GROUPED || (path == MOE_PATH_AUTO && auto_grouped);
  // MX routed weights with 8- or 4-bit activations run on the scaled MFMA
  const bool mx_w = L.wfmt == W_MXFP4 || L.wfmt == W_MXFP8;
  const int mx_bits = mx_w && (L.afmt == A_FP8_TOKEN || L.afmt == A_MXFP8) ? 8 : (mx_w && L.afmt == A_MXFP4 ? 4 : 0);
  p.grouped = want && plan_group(L.wfmt, L.H, L.I, 64, mx_bits, p.gu_rg) &&
              plan_group(sfmt, L.H, Ish, 64, 0, p.gu_sg) &&
              plan_group(L.wfmt, L.I, L.H, 128, mx_bits, p.dn_rg) &&
              plan_group(sfmt, Ish, L.H, 128, 0, p.dn_sg);
  if (p.grouped) {
    auto gbound = [&](const GroupMap& g, int units) {
      return (int64_t)units * g.steps * (g.cw + (int64_t)g.ct * g.NG);
    };
    if (gbound(p.gu_rg, ur) + gbound(p.gu_sg, us) > (1ll << 30) || gbound(p.dn_rg, ur) + gbound(p.dn_sg, us) > (1ll << 30))
      p.grouped = false;
  }
  if (p.grouped) {
    const size_t gemv_tiles[4] = {p.gu_tile, p.dn_tile, p.gu_lds, p.dn_lds};
    auto gtile = [&](const GroupMap& r, const GroupMap& s) {
      return align_up(2 * std::max(group_buf_bytes(r), L.has_shared ? group_buf_bytes(s) : 0), 16) + kGWeightLds;
    };
    p.gu_tile = gtile(p.gu_rg, p.gu_sg);
    p.dn_tile = gtile(p.dn_rg, p.dn_sg);
    p.gu_lds = p.list_bytes + p.gu_tile;
    p.dn_lds = p.list_bytes + p.dn_tile;
    // two workgroups per compute unit, or the GEMV kernels (their LDS stays within 64 KB)
    if (std::max(p.gu_lds, p.dn_lds) > (size_t)kGroupedLdsMax) {
      p.grouped = false;
      p.gu_tile = gemv_tiles[0];
      p.dn_tile = gemv_tiles[1];
      p.gu_lds = gemv_tiles[2];
      p.dn_lds = gemv_tiles[3];
    }
  }
  return true;
}

// Workgroups of a G-workgroup expert launch that walk the shared expert: its share of
// the summed cost, with the routed cost bounded by min(E, T*k) one-group experts (the
// routing is not known on the host). At least one workgroup each. Costs per class:
// units of NG tokens, `steps` steps each, a step costing cw + ct * tokens.
struct CostQ {
  int NG, steps, cw, ct;
};
// The split weighs workgroups as the kernels do: the first ncu blocks 16, later ones
// late16 (shared workgroups come first, so they are all full-weight ones when the shared
// share stays under ncu blocks).
// In pair mode the routed units hold one token each, the shared ones up to NG. With
// block-scaled shared weights (FP4 / FP8) a unit decodes each weight piece once for all
// its tokens, so a unit's tokens after the first cost 3/5 of the token term (graph-timed
// sweep of the shared workgroup count on the Flint W4A16 layer at T = 2..8: 1.2 us per
// layer at T = 8; with BF16 shared weights nothing is amortized and the term stays).
int shared_wgs(const moe_layer_t& L, int T, const CostQ& s, const CostQ& r, int G, int ncu, int late16,
               bool pair_mode = false) {
  if (!L.has_shared || G < 2) return 0;
  const int64_t units = (T + s.NG - 1) / s.NG;
  const bool amortized = pair_mode && L.shared_wfmt != MOE_W_BF16;
  const int64_t cs = amortized ? (int64_t)s.steps * (5 * (s.cw + s.ct) * units + 3 * (int64_t)s.ct * (T - units)) / 5
                               : (int64_t)s.steps * (s.cw * units + (int64_t)s.ct * T);
  const int64_t pairs = (int64_t)T * L.k, ur = pair_mode ? pairs : std::min<int64_t>(L.E, pairs);
  const int64_t cr = (int64_t)r.steps * (r.cw * ur + r.ct * pairs);
  const int64_t W = 16 * (int64_t)std::min(G, ncu) + (int64_t)late16 * std::max(0, G - ncu);
  const int64_t g = (W * cs + 8 * (cs + cr)) / (16 * (cs + cr));
  return (int)std::min<int64_t>(std::max<int64_t>(g, 1), std::min(G, ncu) - 1);
}

// Positions of one cost (pair and token modes) over G workgroups, the first n1 of which
// are dispatched in the first round (one per compute unit). Per-workgroup timestamps on
// the Flint W4A16 layer at T = 8 put the second-round workgroups' start about 0.8 of a
// row-step later and their steps about 15 % slower. The split takes the whole numbers of
// positions per round that minimize the later finish: q2 (+1) per second-round
// workgroup, the rest over the first round.
void split_rounds(ExpertArgs& x, int A, int G, int n1) {
  n1 = std::min(n1, G);
  const int n2 = G - n1;
  auto fill = [&](int A1) {
    x.pn1 = n1;
    x.pq1 = n1 ? A1 / n1 : 0;
    x.pr1 = n1 ? A1 - x.pq1 * n1 : 0;
    const int A2 = A - A1;
    x.pq2 = n2 ? A2 / n2 : 0;
    x.pr2 = n2 ? A2 - x.pq2 * n2 : 0;
  };
  if (n1 == 0 || n2 == 0) { fill(n2 == 0 ? A : 0); return; }
  double best = 1e30;
  int best_A1 = A;
  for (int q2 = 0; q2 <= (A + n2 - 1) / n2; ++q2) {
    const int A2 = std::min(A, n2 * q2), A1 = A - A2;
    const double t1 = A1 > 0 ? (double)((A1 + n1 - 1) / n1) : 0.0;
    const double t2 = A2 > 0 ? 0.8 + 1.15 * (double)((A2 + n2 - 1) / n2) : 0.0;
    const double t = std::max(t1, t2);
    if (t < best) { best = t; best_A1 = A1; }
  }
  fill(best_A1);
}

struct WsLayout {
  size_t logits, h, hq_codes, hq_scales, hq_scale, o, total;
  int hs;
};

WsLayout ws_layout(const moe_layer_t& L, int maxT) {
  WsLayout w{};
  const int Ish = L.has_shared ? L.I_shared : 0;
  const size_t Pr = (size_t)maxT * L.k, Pt = Pr + (L.has_shared ? maxT : 0);
  w.hs = std::max(L.I, Ish);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off = align_up(off + bytes); return at; };
  w.logits = take(8 * (size_t)maxT * L.E);   // logits (keys), then bare logits (selection-only bias)
  w.h = take(4 * Pt * w.hs);
  const size_t qrow = (L.afmt == A_NVFP4_4O6 || L.afmt == A_MXFP4) ? L.I / 2
                      : ((L.afmt == A_FP8_TOKEN || L.afmt == A_MXFP8) ? L.I : 0);
  w.hq_codes = take(Pr * qrow);
  w.hq_scales = take(L.afmt == A_NVFP4_4O6 ? Pr * (L.I / 16)
                     : ((L.afmt == A_MXFP4 || L.afmt == A_MXFP8) ? Pr * (L.I / 32) : 0));
  w.hq_scale = take(4 * Pr);
  w.o = take(4 * Pt * L.H);
  w.total = off;
  return w;
}

// Every violated constraint, or "" if none.
std::string check_layer(const moe_layer_t* L, int max_tokens) {
  if (!L) return "layer pointer is NULL";
  std::string why;
  auto add = [&](const std::string& s) { why += (why.empty() ? "" : "; ") + s; };
  char b[256];
  if (L->H < 32 || L->H % 32) { snprintf(b, sizeof b, "H=%d must be a positive multiple of 32", L->H); add(b); }
  if (L->I < 32 || L->I % 32) { snprintf(b, sizeof b, "I=%d must be a positive multiple of 32", L->I); add(b); }
  if (L->E < 1 || L->E > kMaxE) { snprintf(b, sizeof b, "E=%d must be in [1, %d]", L->E, kMaxE); add(b); }
  if (L->k < 1 || L->k > std::min(std::max(L->E, 1), kMaxK)) {
    snprintf(b, sizeof b, "k=%d must be in [1, min(E, %d)]", L->k, kMaxK); add(b);
  }
  if (L->has_shared != 0 && L->has_shared != 1) add("has_shared must be 0 or 1");
  if (L->router_score != MOE_SCORE_SIGMOID && L->router_score != MOE_SCORE_SOFTMAX) {
    snprintf(b, sizeof b, "router_score=%d is not a moe_score_t", L->router_score); add(b);
  }
  if (L->bias_select_only != 0 && L->bias_select_only != 1) add("bias_select_only must be 0 or 1");
  if (L->has_shared == 1 && (L->I_shared < 32 || L->I_shared % 32)) {
    snprintf(b, sizeof b, "I_shared=%d must be a positive multiple of 32", L->I_shared); add(b);
  }
  if (max_tokens < 1 || max_tokens > kMaxTokens) {
    snprintf(b, sizeof b, "max_tokens=%d must be in [1, %d]", max_tokens, kMaxTokens); add(b);
  }
  const bool wf_ok = valid_wfmt(L->wfmt), sf_ok = valid_wfmt(L->shared_wfmt);
  if (!wf_ok) { snprintf(b, sizeof b, "unknown wfmt %d", L->wfmt); add(b); }
  if (L->has_shared == 1 && !sf_ok) { snprintf(b, sizeof b, "unknown shared_wfmt %d", L->shared_wfmt); add(b); }
  if (L->afmt < MOE_A_BF16 || L->afmt > MOE_A_MXFP8) { snprintf(b, sizeof b, "unknown afmt %d", L->afmt); add(b); }
  if (L->afmt == MOE_A_NVFP4_4O6 && L->wfmt != MOE_W_NVFP4) add("afmt NVFP4_4O6 needs NVFP4 routed weights");
  if (L->afmt == MOE_A_FP8_TOKEN && L->wfmt != MOE_W_MXFP4 && L->wfmt != MOE_W_MXFP8)
    add("afmt FP8_TOKEN needs MXFP4 or MXFP8 routed weights");
  if ((L->afmt == MOE_A_MXFP4 || L->afmt == MOE_A_MXFP8) && L->wfmt != MOE_W_MXFP4 && L->wfmt != MOE_W_MXFP8)
    add("afmt MXFP4 / MXFP8 needs MXFP4 or MXFP8 routed weights");
  if (L->has_shared == 1 && wf_ok && sf_ok && L->shared_wfmt != L->wfmt && L->shared_wfmt != MOE_W_BF16)
    add("the shared expert must use the routed format or BF16");
  if (!L->router_w) add("router_w is NULL");
  else if (!aligned(L->router_w, 16)) add("router_w must be 16-byte aligned");
  auto check_w = [&](const moe_weights_t& w, int fmt, const char* name) {
    if (!w.codes) { snprintf(b, sizeof b, "%s.codes is NULL", name); add(b); }
    else if (!aligned(w.codes, 16)) { snprintf(b, sizeof b, "%s.codes must be 16-byte aligned", name); add(b); }
    if (fmt != MOE_W_BF16 && !w.scales) { snprintf(b, sizeof b, "%s.scales is NULL", name); add(b); }
    if (fmt == MOE_W_NVFP4 && w.scales && !aligned(w.scales, 16)) {
      snprintf(b, sizeof b, "%s.scales must be 16-byte aligned", name); add(b);
    }
    if ((fmt == MOE_W_MXFP4 || fmt == MOE_W_MXFP8) && w.scales && !aligned(w.scales, 4)) {
      snprintf(b, sizeof b, "%s.scales must be 4-byte aligned", name); add(b);
    }
    if (fmt == MOE_W_NVFP4 && !w.gscale) { snprintf(b, sizeof b, "%s.gscale is NULL", name); add(b); }
  };
  if (wf_ok) { check_w(L->w13, L->wfmt, "w13"); check_w(L->w2, L->wfmt, "w2"); }
  if (L->has_shared == 1 && sf_ok) { check_w(L->sh13, L->shared_wfmt, "sh13"); check_w(L->sh2, L->shared_wfmt, "sh2"); }
  if (why.empty()) {
    Plan p;
    if (!make_plan(*L, std::max(1, max_tokens), MOE_PATH_AUTO, p))
      add("no workgroup row mapping fits these sizes (H, I, I_shared) and formats");
  }
  return why;
}

moe_status_t check_or_fail(const moe_layer_t* L, int max_tokens) {
  std::string why = check_layer(L, max_tokens);
  if (!why.empty()) return set_err(L ? MOE_EUNSUPPORTED : MOE_EINVAL, why);
  return MOE_OK;
}

WTensor wtensor(const moe_weights_t& w, int fmt, int rows, int K, int gs_per_expert) {
  WTensor t;
  t.codes = static_cast<const uint8_t*>(w.codes);
  t.scales = fmt == W_BF16 ? nullptr : w.scales;
  t.gscale = fmt == W_NVFP4 ? w.gscale : nullptr;
  t.code_row_bytes = code_row_bytes(fmt, K);
  t.scale_row_bytes = scale_row_bytes(fmt, K);
  t.rows = rows;
  t.K = K;
  t.gs_per_expert = gs_per_expert;
  t.fmt = fmt;
  return t;
}

// Token count the workspace was sized for, recovered from its byte size is not
// possible; callers pass T <= the max_tokens they sized it for, and the check below
// compares against the layout for T itself.
moe_status_t check_ws(const moe_layer_t& L, int T, void* ws, size_t ws_bytes, WsLayout& w) {
  w = ws_layout(L, std::max(1, T));
  if (!ws) return set_err(MOE_EWORKSPACE, "workspace is NULL");
  if (!aligned(ws, kAlign)) return set_err(MOE_EWORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < w.total) {
    char b[160];
    snprintf(b, sizeof b, "workspace has %zu bytes, this call needs %zu", ws_bytes, w.total);
    return set_err(MOE_EWORKSPACE, b);
  }
  return MOE_OK;
}

size_t xq_part(size_t bytes) { return align_up(bytes); }

// Compute units of the current device (cached per device id).
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// The expert kernels are persistent: kWgPerCu resident workgroups per CU (their launch
// bounds allow 2 per CU) split the work units' row-steps between them.
constexpr int kWgPerCu = 2;

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_last_error(void) { return g_err.c_str(); }

moe_status_t moe_layer_check(const moe_layer_t* L, int32_t max_tokens, char* why, size_t why_len) {
  std::string w = check_layer(L, max_tokens);
  if (why && why_len) {
    const size_t n = std::min(w.size(), why_len - 1);
    memcpy(why, w.data(), n);
    why[n] = '\0';
  }
  if (w.empty()) return MOE_OK;
  g_err = w;
  return L ? MOE_EUNSUPPORTED : MOE_EINVAL;
}

size_t moe_workspace_bytes(const moe_layer_t* L, int32_t max_tokens) {
  if (!check_layer(L, max_tokens).empty()) return 0;
  return ws_layout(*L, max_tokens).total;
}

size_t moe_xq_bytes(const moe_layer_t* L, int32_t T) {
  if (!L || T <= 0) return 0;
  if (L->afmt == MOE_A_NVFP4_4O6)
    return xq_part((size_t)T * L->H / 2) + xq_part((size_t)T * L->H / 16) + xq_part(4 * (size_t)T);
  if (L->afmt == MOE_A_FP8_TOKEN) return xq_part((size_t)T * L->H) + xq_part(4 * (size_t)T);
  if (L->afmt == MOE_A_MXFP4) return xq_part((size_t)T * L->H / 2) + xq_part((size_t)T * L->H / 32);
  if (L->afmt == MOE_A_MXFP8) return xq_part((size_t)T * L->H) + xq_part((size_t)T * L->H / 32);
  return 0;
}

moe_status_t moe_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return set_err(MOE_EINVAL, "workspace is NULL");
  if (!aligned(ws, 16) || ws_bytes % 16) return set_err(MOE_EINVAL, "workspace must be 16-byte aligned and sized");
  if (launch_fill_zero(ws, ws_bytes, stream) != hipSuccess) return set_err(MOE_ELAUNCH, "fill kernel launch failed");
  return MOE_OK;
}

}  // extern "C"

namespace {

// Router GEMV (+ token quantization) and, if `topk`, the top-k launch.
// dry: check the arguments only.
// RMSNorm before the layer (moe_forward_fused): resid / gamma / eps, x written to x_out.
struct NormIn {
  const uint16_t* resid = nullptr;
  const uint16_t* gamma = nullptr;
  float eps = 0.0f;
  uint16_t* x_out = nullptr;
};

moe_status_t enqueue_route(const moe_layer_t* L, const uint16_t* x_bf16, int32_t T, int32_t* topk_ids,
                           float* topk_w, void* xq, void* ws, size_t ws_bytes, bool topk, bool dry,
                           hipStream_t stream, const NormIn& nin = NormIn{}) {
  moe_status_t st = check_or_fail(L, std::max(1, T));
  if (st != MOE_OK) return st;
  if (T < 0) return set_err(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return MOE_OK;
  std::string bad;
  if (!x_bf16 || !aligned(x_bf16, 16)) bad += "x_bf16 must be non-NULL and 16-byte aligned; ";
  if (!topk_ids) bad += "topk_ids is NULL; ";
  if (!topk_w) bad += "topk_w is NULL; ";
  if (L->afmt != MOE_A_BF16 && (!xq || !aligned(xq, kAlign))) bad += "xq must be non-NULL and 256-byte aligned; ";
  if (!bad.empty()) return set_err(MOE_EINVAL, bad);
  WsLayout w;
  if ((st = check_ws(*L, T, ws, ws_bytes, w)) != MOE_OK) return st;
  if (dry) return MOE_OK;
  uint8_t* base = static_cast<uint8_t*>(ws);
  RouteArgs a{};
  a.x = x_bf16;
  a.wr = L->router_w;
  a.bias = L->router_bias;
  a.T = T; a.H = L->H; a.E = L->E; a.k = L->k; a.afmt = L->afmt;
  a.softmax = L->router_score == MOE_SCORE_SOFTMAX;
  // bias for selection only: the bare logits go to the second half of the logits area
  a.raw = L->router_bias && L->bias_select_only ? reinterpret_cast<float*>(base + w.logits) + (size_t)T * L->E
                                                : nullptr;
  // decode sizes: one token per workgroup and enough experts per workgroup to keep the
  // launch near 1024 workgroups (graph-timed on the Flint layers: the latency of a
  // workgroup grows with its loads per lane, fastest at 1024 short workgroups)
  a.TT = T <= kRouteSmallT ? 1 : kRouteTT;
  a.ET = T <= 4 ? 1 : (T <= 8 ? 2 : 4);
  a.n_tt = (T + a.TT - 1) / a.TT;
  a.n_et = (L->E + a.ET - 1) / a.ET;
  a.logits = reinterpret_cast<float*>(base + w.logits);
  a.ids = topk_ids;
  a.w = topk_w;
  int n_quant = 0;
  if (L->afmt != MOE_A_BF16) {
    uint8_t* q = static_cast<uint8_t*>(xq);
    a.xq_codes = q;
    if (L->afmt == MOE_A_NVFP4_4O6) {
      a.xq_scales = q + xq_part((size_t)T * L->H / 2);
      a.xq_scale = reinterpret_cast<float*>(a.xq_scales + xq_part((size_t)T * L->H / 16));
    } else if (L->afmt == MOE_A_FP8_TOKEN) {
      a.xq_scale = reinterpret_cast<float*>(q + xq_part((size_t)T * L->H));
    } else {   // MX: codes, then E8M0 scales
      a.xq_scales = q + xq_part((size_t)T * L->H / (L->afmt == MOE_A_MXFP4 ? 2 : 1));
    }
    n_quant = T;
  }
  if (nin.resid) {   // the per-token workgroups also write the normalized tokens
    a.resid = nin.resid;
    a.gamma = nin.gamma;
    a.eps = nin.eps;
    a.x_out = nin.x_out;
    n_quant = T;
  }
  if (launch_route(a, n_quant, topk, stream) != hipSuccess) return set_err(MOE_ELAUNCH, "route kernel launch failed");
  return MOE_OK;
}

// Whether the experts of a T-token call run the GEMV kernels in pair mode, where the
// gate/up kernel can do the routing itself (for E <= 64 * kFusedTopkSlots).
bool pair_mode_plan(const moe_layer_t& L, int T, int path) {
  Plan p;
  return T * L.k <= kPairMax && L.E <= 64 * kFusedTopkSlots && make_plan(L, T, path, p) && !p.grouped;
}

// Expert kernels (and combine); with fused_topk the gate/up kernel selects the experts
// from the router logits in the workspace and writes topk_ids / topk_w itself.
moe_status_t enqueue_experts(const moe_layer_t* L, const uint16_t* x_bf16, const void* xq, int32_t T,
                             const int32_t* topk_ids, const float* topk_w, uint16_t* y_bf16, void* ws,
                             size_t ws_bytes, const moe_debug_t* dbg, bool fused_topk, bool dry,
                             hipStream_t stream, const uint16_t* resid = nullptr) {
  moe_status_t st = check_or_fail(L, std::max(1, T));
  if (st != MOE_OK) return st;
  if (T < 0) return set_err(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return MOE_OK;
  std::string bad;
  if (!x_bf16 || !aligned(x_bf16, 16)) bad += "x_bf16 must be non-NULL and 16-byte aligned; ";
  if (!topk_ids) bad += "topk_ids is NULL; ";
  if (!topk_w) bad += "topk_w is NULL; ";
  if (!y_bf16) bad += "y_bf16 is NULL; ";
  if (L->afmt != MOE_A_BF16 && (!xq || !aligned(xq, kAlign))) bad += "xq must be non-NULL and 256-byte aligned; ";
  if (dbg && dbg->hq_codes && L->afmt == MOE_A_BF16) bad += "dbg->hq_codes needs a quantized afmt; ";
  if (dbg && dbg->hq_codes && L->afmt != MOE_A_BF16 &&
      (((L->afmt == MOE_A_NVFP4_4O6 || L->afmt == MOE_A_FP8_TOKEN) && !dbg->hq_scale) ||
       (L->afmt != MOE_A_FP8_TOKEN && !dbg->hq_scales)))
    bad += "dbg->hq_codes needs hq_scale (NVFP4, FP8 per token) and hq_scales (NVFP4, MX); ";
  if (dbg && dbg->hq_codes && !aligned(dbg->hq_codes, 16)) bad += "dbg->hq_codes must be 16-byte aligned; ";
  if (!bad.empty()) return set_err(MOE_EINVAL, bad);
  WsLayout w;
  if ((st = check_ws(*L, T, ws, ws_bytes, w)) != MOE_OK) return st;
  const int resident = kWgPerCu * device_cus();
  const int path = dbg ? dbg->path : MOE_PATH_AUTO;
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GROUPED) return set_err(MOE_EINVAL, "dbg->path is not a moe_path_t");
  Plan p;
  if (!make_plan(*L, T, path, p)) return set_err(MOE_EUNSUPPORTED, "no launch plan");
  if (path == MOE_PATH_GROUPED && !p.grouped)
    return set_err(MOE_EUNSUPPORTED,
                   "grouped kernels need K and rows that tile (H, I multiples of the stage and tile sizes) and at "
                   "most 80 KB of LDS per workgroup (the expert tables grow with T * k and E)");
  if (fused_topk && (p.grouped || T * L->k > kPairMax)) return set_err(MOE_EINVAL, "fused routing needs pair mode");
  if (dry) return MOE_OK;
  uint8_t* base = static_cast<uint8_t*>(ws);
  const int Ish = L->has_shared ? L->I_shared : L->I;
  const int sfmt = L->has_shared ? L->shared_wfmt : L->wfmt;
  ExpertArgs a{};
  a.x = x_bf16;
  if (L->afmt != MOE_A_BF16) {
    const uint8_t* q = static_cast<const uint8_t*>(xq);
    a.xq_codes = q;
    if (L->afmt == MOE_A_NVFP4_4O6) {
      a.xq_scales = q + xq_part((size_t)T * L->H / 2);
      a.xq_scale = reinterpret_cast<const float*>(a.xq_scales + xq_part((size_t)T * L->H / 16));
    } else if (L->afmt == MOE_A_FP8_TOKEN) {
      a.xq_scale = reinterpret_cast<const float*>(q + xq_part((size_t)T * L->H));
    } else {   // MX: codes, then E8M0 scales
      a.xq_scales = q + xq_part((size_t)T * L->H / (L->afmt == MOE_A_MXFP4 ? 2 : 1));
    }
  }
  a.ids = topk_ids;
  a.topk_w = topk_w;
  a.T = T; a.H = L->H; a.I = L->I; a.Ish = Ish; a.E = L->E; a.k = L->k;
  a.inv_k = 1.0f / (float)L->k;
  a.has_shared = L->has_shared; a.afmt = L->afmt;
  a.max_slots = p.max_slots;
  a.h = reinterpret_cast<float*>(base + w.h);
  a.hs = w.hs;
  a.hq_codes = base + w.hq_codes;
  a.hq_scales = base + w.hq_scales;
  a.hq_scale = reinterpret_cast<float*>(base + w.hq_scale);
  a.o = reinterpret_cast<float*>(base + w.o);
  a.y = y_bf16;
  a.resid = resid;
  if (dbg) {
    a.dbg_h = dbg->h;
    a.dbg_codes = dbg->hq_codes;
    a.dbg_scales = dbg->hq_scales;
    a.dbg_scale = dbg->hq_scale;
  }
  a.lds_list_bytes = (int)p.list_bytes;

  ExpertArgs gu = a, dn = a;
  gu.rw = wtensor(L->w13, L->wfmt, 2 * L->I, L->H, 2);
  gu.sw = wtensor(L->has_shared ? L->sh13 : L->w13, sfmt, 2 * Ish, L->H, 2);
  gu.rmap = p.gu_r;
  gu.smap = p.gu_s;
  gu.lds_act_bytes = (int)p.gu_tile;
  dn.rw = wtensor(L->w2, L->wfmt, L->H, L->I, 1);
  dn.sw = wtensor(L->has_shared ? L->sh2 : L->w2, sfmt, L->H, Ish, 1);
  dn.rmap = p.dn_r;
  dn.smap = p.dn_s;
  dn.lds_act_bytes = (int)p.dn_tile;
  // persistent launches: every workgroup takes a share of its class's cost, the
  // second-round blocks (dispatched once every compute unit holds one) a smaller one
  const int gu_grid = resident, dn_grid = resident;
  const int ncu = device_cus();
  gu.ncu = dn.ncu = ncu;
  gu.late16 = p.grouped ? 16 : kLateGateup16;
  dn.late16 = p.grouped ? 16 : kLateDown16;
  const int Ish_ = L->has_shared ? L->I_shared : L->I;
  gu.grouped = dn.grouped = p.grouped ? 1 : 0;
  if (p.grouped) {
    gu.rgm = p.gu_rg; gu.sgm = p.gu_sg;
    dn.rgm = p.dn_rg; dn.sgm = p.dn_sg;
    auto q = [](const GroupMap& g) { return CostQ{g.NG, g.steps * g.NS, g.cw / g.NS, g.ct / g.NS}; };
    gu.sh_wgs = shared_wgs(*L, T, q(p.gu_sg), q(p.gu_rg), gu_grid, ncu, gu.late16);
    dn.sh_wgs = shared_wgs(*L, T, q(p.dn_sg), q(p.dn_rg), dn_grid, ncu, dn.late16);
  } else {
    const bool pm = T * L->k <= kPairMax;
    gu.pair_mode = dn.pair_mode = pm ? 1 : 0;
    if (fused_topk) {
      gu.fuse_topk = 1;
      gu.logits = reinterpret_cast<const float*>(base + w.logits);
      gu.ids_out = const_cast<int32_t*>(topk_ids);
      gu.w_out = const_cast<float*>(topk_w);
      gu.raw = L->router_bias && L->bias_select_only
                   ? reinterpret_cast<const float*>(base + w.logits) + (size_t)T * L->E : nullptr;
      gu.softmax = L->router_score == MOE_SCORE_SOFTMAX;
    }
    // token mode: items of (token, row-step) over all of the token's experts, writing y.
    // Wide items of G rows, whose experts the four waves split (an item issues two
    // experts' loads per lane instead of k + 1), while they fit one per resident workgroup
    // and give at least half a workgroup per compute unit: one or two tokens. Past that,
    // items of RS rows under the same floor (graph-timed on the Flint W4A16 layer: at
    // 4 and 8 tokens a workgroup's one burst of k + 1 experts beats wide items streamed
    // two at a time, 11.3 against 12.3 us and 15.2 against 17.4 us); else the per-pair
    // walk and the combine launch.
    {
      const int full = L->H / p.dn_r.RS, wide = L->H / p.dn_r.G;
      int tm = 0;
      if (pm && p.token) {
        if (T * wide <= dn_grid && 2 * T * wide >= ncu && 4 * p.dn_r.G <= 2 * kWinRows) tm = 2;
        else if (2 * T * full >= ncu) tm = 1;
      }
      dn.token_mode = tm;
      dn.tok_items = tm == 2 ? wide : full;
      dn.tok_inv = 1.0f / (float)dn.tok_items;
    }
    auto q = [](const GemvMap& m, int steps) { return CostQ{m.NG, steps, m.cw, m.ct}; };
    // The shared expert's token groups each walk all of its rows. With groups of equal
    // size and a multiple of 8 x groups shared workgroups (all in the first round), group
    // g's workgroup b + g x (count / groups) walks the same rows as workgroup b of group 0,
    // at the same time and on the same XCD (blocks go round-robin over the 8 XCDs), so
    // the later groups' reads hit that XCD's L2 instead of memory.
    auto xcd_align = [&](int g, const GemvMap& m, int grid) {
      const int groups = (T + m.NG - 1) / m.NG, step = 8 * groups;
      if (groups < 2 || T % m.NG || g < step) return g;
      int r = (g + step / 2) / step * step;
      while (r > std::min(grid, ncu) - 1) r -= step;
      return r >= step ? r : g;
    };
    gu.sh_wgs = xcd_align(shared_wgs(*L, T, q(p.gu_s, Ish_ / (p.gu_s.RS / 2)), q(p.gu_r, L->I / (p.gu_r.RS / 2)),
                                     gu_grid, ncu, gu.late16, pm),
                          p.gu_s, gu_grid);
    dn.sh_wgs = dn.token_mode ? 0
                              : xcd_align(shared_wgs(*L, T, q(p.dn_s, L->H / p.dn_s.RS), q(p.dn_r, L->H / p.dn_r.RS),
                                                     dn_grid, ncu, dn.late16, pm),
                                          p.dn_s, dn_grid);
    // pair and token modes: every position of the class costs the same
    if (pm) {
      split_rounds(gu, T * L->k * p.gu_r.steps, gu_grid - gu.sh_wgs, std::max(0, ncu - gu.sh_wgs));
      if (!dn.token_mode)
        split_rounds(dn, T * L->k * p.dn_r.steps, dn_grid - dn.sh_wgs, std::max(0, ncu - dn.sh_wgs));
    }
    if (dn.token_mode) split_rounds(dn, T * dn.tok_items, dn_grid, ncu);
  }
  if (launch_experts(gu, gu_grid, p.gu_lds, dn, dn_grid, p.dn_lds, stream) != hipSuccess)
    return set_err(MOE_ELAUNCH, "expert kernel launch failed");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_route(const moe_layer_t* L, const uint16_t* x_bf16, int32_t T, int32_t* topk_ids,
                       float* topk_w, void* xq, void* ws, size_t ws_bytes, hipStream_t stream) {
  return enqueue_route(L, x_bf16, T, topk_ids, topk_w, xq, ws, ws_bytes, true, false, stream);
}

moe_status_t moe_expert_forward(const moe_layer_t* L, const uint16_t* x_bf16, const void* xq, int32_t T,
                                const int32_t* topk_ids, const float* topk_w, uint16_t* y_bf16,
                                void* ws, size_t ws_bytes, const moe_debug_t* dbg, hipStream_t stream) {
  return enqueue_experts(L, x_bf16, xq, T, topk_ids, topk_w, y_bf16, ws, ws_bytes, dbg, false, false, stream);
}

moe_status_t moe_forward(const moe_layer_t* L, const uint16_t* x_bf16, int32_t T, int32_t* topk_ids,
                         float* topk_w, void* xq, uint16_t* y_bf16, void* ws, size_t ws_bytes,
                         const moe_debug_t* dbg, hipStream_t stream) {
  moe_status_t st = check_or_fail(L, std::max(1, T));
  if (st != MOE_OK) return st;
  if (T < 0) return set_err(MOE_EINVAL, "T must be >= 0");
  if (T == 0) return MOE_OK;
  const int path = dbg ? dbg->path : MOE_PATH_AUTO;
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GROUPED) return set_err(MOE_EINVAL, "dbg->path is not a moe_path_t");
  const bool fused = pair_mode_plan(*L, T, path);
  // every check of both halves before the first launch
  if ((st = enqueue_route(L, x_bf16, T, topk_ids, topk_w, xq, ws, ws_bytes, !fused, true, stream)) != MOE_OK ||
      (st = enqueue_experts(L, x_bf16, xq, T, topk_ids, topk_w, y_bf16, ws, ws_bytes, dbg, fused, true, stream)) !=
          MOE_OK)
    return st;
  if ((st = enqueue_route(L, x_bf16, T, topk_ids, topk_w, xq, ws, ws_bytes, !fused, false, stream)) != MOE_OK)
    return st;
  return enqueue_experts(L, x_bf16, xq, T, topk_ids, topk_w, y_bf16, ws, ws_bytes, dbg, fused, false, stream);
}

moe_status_t moe_forward_fused(const moe_layer_t* L, const moe_norm_t* norm, const uint16_t* resid_in, int32_t T,
                               uint16_t* x_out, int32_t* topk_ids, float* topk_w, void* xq, uint16_t* resid_out,
                               void* ws, size_t ws_bytes, const moe_debug_t* dbg, hipStream_t stream) {
  moe_status_t st = check_or_fail(L, std::max(1, T));
  if (st != MOE_OK) return st;
  if (T < 0) return set_err(MOE_EINVAL, "T must be >= 0");
  std::string bad;
  if (!norm) bad += "norm is NULL; ";
  else {
    if (!norm->gamma || !aligned(norm->gamma, 16)) bad += "norm->gamma must be non-NULL and 16-byte aligned; ";
    if (!(norm->eps >= 0.0f) || !(norm->eps < 3.4e38f)) bad += "norm->eps must be finite and >= 0; ";
  }
  if (T > 0) {
    if (!resid_in || !aligned(resid_in, 16)) bad += "resid_in must be non-NULL and 16-byte aligned; ";
    if (!x_out || !aligned(x_out, 16)) bad += "x_out must be non-NULL and 16-byte aligned; ";
    if (!resid_out) bad += "resid_out is NULL; ";
    // x_out is written while the router reads resid_in, in the same launch
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(resid_in), x0 = reinterpret_cast<uintptr_t>(x_out);
    const uintptr_t n = (uintptr_t)T * L->H * 2;
    if (resid_in && x_out && a0 < x0 + n && x0 < a0 + n) bad += "x_out must not overlap resid_in; ";
  }
  if (!bad.empty()) return set_err(MOE_EINVAL, bad);
  if (T == 0) return MOE_OK;
  const int path = dbg ? dbg->path : MOE_PATH_AUTO;
  if (path < MOE_PATH_AUTO || path > MOE_PATH_GROUPED) return set_err(MOE_EINVAL, "dbg->path is not a moe_path_t");
  const bool fused = pair_mode_plan(*L, T, path);
  const NormIn nin{resid_in, norm->gamma, norm->eps, x_out};
  // every check of both halves before the first launch
  if ((st = enqueue_route(L, x_out, T, topk_ids, topk_w, xq, ws, ws_bytes, !fused, true, stream, nin)) != MOE_OK ||
      (st = enqueue_experts(L, x_out, xq, T, topk_ids, topk_w, resid_out, ws, ws_bytes, dbg, fused, true, stream,
                            resid_in)) != MOE_OK)
    return st;
  if ((st = enqueue_route(L, x_out, T, topk_ids, topk_w, xq, ws, ws_bytes, !fused, false, stream, nin)) != MOE_OK)
    return st;
  return enqueue_experts(L, x_out, xq, T, topk_ids, topk_w, resid_out, ws, ws_bytes, dbg, fused, false, stream,
                         resid_in);
}

}  // extern "C"

// ------------------------------------------------------------ allocation-free variant
// moe_forward_noalloc runs moe_forward on a workspace that lives in this library's own
// device memory: a file-scope array, one copy per GPU, kept until the process ends. Host
// code never passes the array's name to a kernel (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device, with that device
// current.
namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, or NULL with the error set.
void* scratch_for_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    set_err(MOE_ELAUNCH, "no current HIP device");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_err(MOE_ELAUNCH, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

moe_status_t moe_forward_noalloc(const moe_layer_t* L, const uint16_t* x_bf16, int32_t T, int32_t* topk_ids,
                                 float* topk_w, void* xq, uint16_t* y_bf16, const moe_debug_t* dbg,
                                 hipStream_t stream) {
  moe_status_t st = check_or_fail(L, std::max(1, T));
  if (st != MOE_OK) return st;
  if (T < 0) return set_err(MOE_EINVAL, "T must be >= 0");
  const size_t need = ws_layout(*L, std::max(1, T)).total;
  if (need > kScratchBytes) {
    char b[200];
    snprintf(b, sizeof b, "this call needs %zu bytes of workspace; the library's static scratch holds %zu "
             "(use moe_forward with a caller workspace)", need, kScratchBytes);
    return set_err(MOE_EWORKSPACE, b);
  }
  if (T == 0) return MOE_OK;
  void* ws = scratch_for_current_device();
  if (!ws) return MOE_ELAUNCH;
  return moe_forward(L, x_bf16, T, topk_ids, topk_w, xq, y_bf16, ws, kScratchBytes, dbg, stream);
}

moe_status_t moe_requant_mxfp4(const uint16_t* w_bf16, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream) {
  std::string bad;
  if (rows < 0) bad += "rows must be >= 0; ";
  if (cols <= 0 || cols % 32) bad += "cols must be a positive multiple of 32; ";
  if (rows > 0) {
    if (!w_bf16 || !aligned(w_bf16, 16)) bad += "w_bf16 must be non-NULL and 16-byte aligned; ";
    if (!codes || !aligned(codes, 16)) bad += "codes must be non-NULL and 16-byte aligned; ";
    if (!scales) bad += "scales is NULL; ";
  }
  if (!bad.empty()) return set_err(MOE_EINVAL, bad);
  if (rows == 0) return MOE_OK;
  if (launch_requant_mxfp4(w_bf16, rows * (cols / 32), codes, scales, stream) != hipSuccess)
    return set_err(MOE_ELAUNCH, "requant kernel launch failed");
  return MOE_OK;
}

moe_status_t moe_requant_fp8_block_mxfp4(const uint8_t* w_fp8, const float* block_scales, int64_t rows, int32_t cols,
                                         int32_t block_rows, int32_t block_cols, uint8_t* codes, uint8_t* scales,
                                         hipStream_t stream) {
  std::string bad;
  if (rows < 0) bad += "rows must be >= 0; ";
  if (cols <= 0 || cols % 32) bad += "cols must be a positive multiple of 32; ";
  if (block_rows <= 0 || block_cols <= 0) bad += "block_rows and block_cols must be positive; ";
  if (rows > 0 && cols > 0 && rows > (int64_t)0x7FFFFFFF * 32 / cols) bad += "at most 2^31 blocks of 32 per call; ";
  if (rows > 0) {
    if (!w_fp8 || !aligned(w_fp8, 16)) bad += "w_fp8 must be non-NULL and 16-byte aligned; ";
    if (!block_scales) bad += "block_scales is NULL; ";
    if (!codes || !aligned(codes, 16)) bad += "codes must be non-NULL and 16-byte aligned; ";
    if (!scales) bad += "scales is NULL; ";
  }
  if (!bad.empty()) return set_err(MOE_EINVAL, bad);
  if (rows == 0) return MOE_OK;
  if (launch_requant_fp8b_mxfp4(w_fp8, block_scales, rows, cols, block_rows, block_cols, codes, scales, stream) !=
      hipSuccess)
    return set_err(MOE_ELAUNCH, "requant kernel launch failed");
  return MOE_OK;
}

moe_status_t moe_requant_mxfp8(const uint16_t* w_bf16, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                               hipStream_t stream) {
  std::string bad;
  if (rows < 0) bad += "rows must be >= 0; ";
  if (cols <= 0 || cols % 32) bad += "cols must be a positive multiple of 32; ";
  if (rows > 0) {
    if (!w_bf16 || !aligned(w_bf16, 16)) bad += "w_bf16 must be non-NULL and 16-byte aligned; ";
    if (!codes || !aligned(codes, 16)) bad += "codes must be non-NULL and 16-byte aligned; ";
    if (!scales) bad += "scales is NULL; ";
  }
  if (!bad.empty()) return set_err(MOE_EINVAL, bad);
  if (rows == 0) return MOE_OK;
  if (launch_requant_mxfp8(w_bf16, rows * (cols / 32), codes, scales, stream) != hipSuccess)
    return set_err(MOE_ELAUNCH, "requant kernel launch failed");
  return MOE_OK;
}

moe_status_t moe_requant_nvfp4(const uint16_t* w_bf16, int32_t ntensors, int64_t rows, int32_t cols,
                               uint8_t* codes, uint8_t* scales, float* gscale, hipStream_t stream) {
  std::string bad;
  if (ntensors < 0 || ntensors > 65535) bad += "ntensors must be in [0, 65535]; ";
  if (rows < 0) bad += "rows must be >= 0; ";
  if (cols <= 0 || cols % 16) bad += "cols must be a positive multiple of 16; ";
  if (rows > 0 && (int64_t)cols * rows / 16 > (int64_t)0x7FFFFFFF) bad += "a tensor may hold at most 2^31 blocks; ";
  if (ntensors > 0 && rows > 0) {
    if (!w_bf16 || !aligned(w_bf16, 16)) bad += "w_bf16 must be non-NULL and 16-byte aligned; ";
    if (!codes || !aligned(codes, 8)) bad += "codes must be non-NULL and 8-byte aligned; ";
    if (!scales) bad += "scales is NULL; ";
    if (!gscale) bad += "gscale is NULL; ";
  }
  if (!bad.empty()) return set_err(MOE_EINVAL, bad);
  if (ntensors == 0 || rows == 0) return MOE_OK;
  if (launch_requant_nvfp4(w_bf16, ntensors, rows * cols, codes, scales, gscale, stream) != hipSuccess)
    return set_err(MOE_ELAUNCH, "requant kernel launch failed");
  return MOE_OK;
}

moe_status_t quantize_nvfp4_4o6(const uint16_t* x_bf16, int32_t rows, int32_t cols, uint8_t* codes,
                                uint8_t* scales, float* gscale, uint8_t* choice, hipStream_t stream) {
  std::string bad;
  if (rows < 0) bad += "rows must be >= 0; ";
  if (cols <= 0 || cols % 16) bad += "cols must be a positive multiple of 16; ";
  if (rows > 0) {
    if (!x_bf16 || !aligned(x_bf16, 16) || (cols % 8)) bad += "x_bf16 must be non-NULL with 16-byte aligned rows; ";
    if (!codes || !aligned(codes, 8)) bad += "codes must be non-NULL and 8-byte aligned; ";
    if (!scales) bad += "scales is NULL; ";
    if (!gscale) bad += "gscale is NULL; ";
  }
  if (!bad.empty()) return set_err(MOE_EINVAL, bad);
  if (rows == 0) return MOE_OK;
  if (launch_quantize_nvfp4(x_bf16, rows, cols, codes, scales, gscale, choice, stream) != hipSuccess)
    return set_err(MOE_ELAUNCH, "quantize kernel launch failed");
  return MOE_OK;
}

}  // extern "C"
