// Work spans of the expert launches: the cost model and where a workgroup's share of a
// class starts and ends.
#pragma once
#include "device.hpp"
#include "plan.hpp"

namespace moe {

// Cost parameters of one class in one kernel.
struct ClassCost {
  int NG, steps, cw, ct;
};

// One workgroup's part of a class: its first position, how many positions it walks,
// and one past the last class row it touches.
struct Span {
  int a0, g0, s0;     // first position (b = 0)
  int e0, n0, rb0;    // expert id, tokens and first class row of expert index a0
  int left;           // positions (row-steps x batches) to walk; 0 = none
  int row_limit;
};

// The expert whose cost block holds cost c, with its prefix values (a = A past the end).
struct Located {
  int a, n, cost, unit, row, id;
};

// Step position (g, s) of cost c in the located expert: the first position whose start
// cost is >= c. Rolls over to the next expert (id unknown: -1) past the expert's last.
__device__ __forceinline__ void place(Located& x, int A, const ClassCost& k, int c, int& g, int& s) {
  g = 0;
  s = 0;
  if (x.a >= A) return;
  const int G = (x.n + k.NG - 1) / k.NG;
  const int rem = c - x.cost;
  const int F = k.steps * (k.cw + k.ct * k.NG);
  g = min(rem / F, G - 1);
  const int cs = k.cw + k.ct * min(k.NG, x.n - g * k.NG);
  s = (rem - g * F + cs - 1) / cs;
  if (s >= k.steps) {
    s = 0;
    if (++g >= G) {
      g = 0;
      ++x.a;
      x.unit += G;
      x.row += x.n;
      x.id = -1;
    }
  }
}

// Span from the located start and end costs (positions walked: start <= p < end).
__device__ __forceinline__ Span make_span(Located lo, Located hi, int A, const ClassCost& k, int c_lo,
                                          int c_hi, int NB) {
  int g0, s0, g1, s1;
  place(lo, A, k, c_lo, g0, s0);
  place(hi, A, k, c_hi, g1, s1);
  Span sp;
  sp.a0 = lo.a; sp.g0 = g0; sp.s0 = s0;
  sp.e0 = lo.id; sp.n0 = lo.n; sp.rb0 = lo.row;
  const int l0 = (lo.unit + g0) * k.steps + s0, l1 = (hi.unit + g1) * k.steps + s1;
  sp.left = l1 > l0 ? (l1 - l0) * NB : 0;
  sp.row_limit = hi.row + g1 * k.NG + (s1 > 0 ? min(k.NG, hi.n - g1 * k.NG) : 0);
  return sp;
}

// How the workgroups of a class weigh against each other: the class starts at launch
// block B0; blocks at or past ncu (one per compute unit) are dispatched in a second round,
// start later and share their compute unit, so they take late16 / 16 of a full share.
struct ShareW {
  int B0, ncu, late16;
};

// Start of workgroup b's share of a class total over G workgroups: floor(total * W(b) /
// W(G)), W the summed weights of the blocks before b (64-bit: total < 2^30, W < 2^21).
__device__ __forceinline__ int share_at(int total, int b, int G, const ShareW& w) {
  if (b >= G) return total;
  auto W = [&](int i) {
    const int g = w.B0 + i;
    return (int64_t)16 * min(g, w.ncu) + (int64_t)w.late16 * max(0, g - w.ncu);
  };
  const int64_t w0 = W(0);
  return (int)((int64_t)total * (W(b) - w0) / (W(G) - w0));
}
// The same through FP32 (no integer division): floor(total * W(b) / W(G)) up to rounding.
// Neighbouring workgroups evaluate the same expression, so the shares still tile
// [0, total) exactly, in order; the last one ends at total.
__device__ __forceinline__ int share_at_f(int total, int b, int G, const ShareW& w) {
  if (b >= G) return total;
  auto W = [&](int i) {
    const int g = w.B0 + i;
    return 16 * min(g, w.ncu) + w.late16 * max(0, g - w.ncu);
  };
  const int w0 = W(0);
  const float f = (float)(W(b) - w0) * __builtin_amdgcn_rcpf((float)(W(G) - w0));
  return min(total, (int)((float)total * f));
}
// x / d for 0 <= x < 2^20 and d >= 1 given inv = 1/d (FP32): (x + 1/2) / d is at least
// 1/(2d) away from an integer, far more than the FP32 error.
__device__ __forceinline__ int div_by(int x, float inv) { return (int)(((float)x + 0.5f) * inv); }
__device__ __forceinline__ void wg_share(int total, int b, int G, const ShareW& w, int& c_lo, int& c_hi) {
  c_lo = share_at(total, b, G, w);
  c_hi = share_at(total, b + 1, G, w);
}

// Workgroup b's positions [l0, l0 + len) of a class whose positions all cost the same,
// in the host's two-round split (see ExpertArgs::pn1).
__device__ __forceinline__ void split_at(int b, int n1, int q1, int r1, int q2, int r2, int& l0, int& len) {
  if (b < n1) {
    l0 = b * q1 + min(b, r1);
    len = q1 + (b < r1 ? 1 : 0);
  } else {
    const int bb = b - n1;
    l0 = n1 * q1 + r1 + bb * q2 + min(bb, r2);
    len = q2 + (bb < r2 ? 1 : 0);
  }
}

// The shared expert's span for workgroup b of G: closed form, no table reads.
__device__ __forceinline__ Span shared_span(int T, const ClassCost& k, int NB, int b, int G, const ShareW& w) {
  const int units = (T + k.NG - 1) / k.NG;
  const int total = k.steps * (k.cw * units + k.ct * T);
  const int c_lo = share_at_f(total, b, G, w), c_hi = share_at_f(total, b + 1, G, w);
  const Located in{0, T, 0, 0, 0, 0}, end{1, T, total, units, T, -1};
  return make_span(c_lo < total ? in : end, c_hi < total ? in : end, 1, k, c_lo, c_hi, NB);
}


}  // namespace moe
