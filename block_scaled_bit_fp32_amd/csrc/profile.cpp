// Opt-in per-kernel device timing (moe_profile_begin / moe_profile_end). Diagnostic:
// meant for measurement runs, not for stream capture. One global session, guarded by a
// mutex; events are created on first use and reused.
#include <hip/hip_runtime_api.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "moe.h"

namespace moe {

namespace {
struct Rec {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_mu;
std::atomic<bool> g_on{false};
std::vector<hipEvent_t> g_pool;   // all events ever created
size_t g_next = 0;                // next unused pool slot in this session
std::vector<Rec> g_recs;
const char* const kNames[] = {"route", "gateup", "down", "quantize_nvfp4", "fill", "topk", "hquant",
                              "combine"};
constexpr int kKinds = 8;
}  // namespace

bool profiling_enabled() { return g_on.load(std::memory_order_relaxed); }

bool profile_events(int kind, hipEvent_t* start, hipEvent_t* stop) {
  std::lock_guard<std::mutex> lk(g_mu);
  while (g_pool.size() < g_next + 2) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return false;
    g_pool.push_back(e);
  }
  *start = g_pool[g_next];
  *stop = g_pool[g_next + 1];
  g_next += 2;
  g_recs.push_back({kind, *start, *stop});
  return true;
}

}  // namespace moe

using namespace moe;

extern "C" {

moe_status_t moe_profile_begin(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.clear();
  g_next = 0;
  g_on.store(true);
  return MOE_OK;
}

int32_t moe_profile_end(moe_kernel_time_t* out, int32_t max_entries) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on.store(false);
  double ms[kKinds] = {0};
  int32_t n[kKinds] = {0};
  for (const Rec& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) continue;
    float t = 0.0f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) continue;
    ms[r.kind] += t;
    n[r.kind] += 1;
  }
  g_recs.clear();
  g_next = 0;
  int32_t k = 0;
  for (int i = 0; i < kKinds && k < max_entries; ++i) {
    if (!out) break;
    out[k].name = kNames[i];
    out[k].launches = n[i];
    out[k].total_ms = ms[i];
    ++k;
  }
  return k;
}

}  // extern "C"
