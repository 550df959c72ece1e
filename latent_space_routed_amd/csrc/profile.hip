// Optional per-kernel timing with HIP events recorded on the launch stream (a measurement aid).
// With timing off (the default) a launch reads one atomic flag and touches no other state; with
// timing on, the event lists are guarded by one lock, so host threads may launch concurrently.
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"

namespace lmoe {
namespace {

struct Pending {
  const char* name;
  hipEvent_t a, b;
};
struct Total {
  int64_t launches = 0;
  double ms = 0.0;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;     // guards everything below
std::string g_only;  // when not empty, the one kernel name that is timed
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
std::map<std::string, Total> g_totals;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

KernelTimer::KernelTimer(const char* n, hipStream_t s) : name(n), stream(s), ev0(nullptr) {
  if (!g_enabled.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_only.empty() && (n == nullptr || g_only != n)) return;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;  // no timing events inside a graph capture
  if (hipStreamIsCapturing(s, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return;
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, s) == hipSuccess) ev0 = e;
}

KernelTimer::~KernelTimer() {
  if (!ev0) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t e = take_event();
  if (e && hipEventRecord(e, stream) == hipSuccess) {
    g_pending.push_back({name, static_cast<hipEvent_t>(ev0), e});
  } else {
    g_pool.push_back(static_cast<hipEvent_t>(ev0));
    if (e) g_pool.push_back(e);
  }
}

}  // namespace lmoe

extern "C" {

void lmoe_profile_enable(int on) { lmoe::g_enabled.store(on != 0, std::memory_order_relaxed); }

void lmoe_profile_only(const char* name) {
  std::lock_guard<std::mutex> lk(lmoe::g_mu);
  lmoe::g_only = name ? name : "";
}

void lmoe_profile_reset(void) {
  std::lock_guard<std::mutex> lk(lmoe::g_mu);
  lmoe::g_totals.clear();
}

lmoe_status lmoe_profile_collect(void) {
  std::lock_guard<std::mutex> lk(lmoe::g_mu);
  lmoe_status st = LMOE_OK;
  for (auto& p : lmoe::g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.b) != hipSuccess || hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) {
      st = LMOE_ERR_HIP;
    } else {
      auto& t = lmoe::g_totals[p.name];
      t.launches += 1;
      t.ms += ms;
    }
    lmoe::g_pool.push_back(p.a);
    lmoe::g_pool.push_back(p.b);
  }
  lmoe::g_pending.clear();
  return st;
}

int lmoe_profile_get(const char* name, int64_t* launches, double* total_ms) {
  if (!name) return 0;
  std::lock_guard<std::mutex> lk(lmoe::g_mu);
  auto it = lmoe::g_totals.find(name);
  if (it == lmoe::g_totals.end()) return 0;
  if (launches) *launches = it->second.launches;
  if (total_ms) *total_ms = it->second.ms;
  return 1;
}

}  // extern "C"
