// Opt-in per-kernel timing: a HIP event pair around each matching launch,
// on the stream the kernel runs on. Off by default; when off a launch pays
// one relaxed atomic load. Durations are resolved when queried.
#include <atomic>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "gs_internal.h"

namespace gs {

namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::atomic<int> g_on{0};
std::mutex g_mu;
std::string g_filter;
std::vector<Rec> g_recs;

bool matches(const char* name) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_filter.empty() || std::strstr(name, g_filter.c_str()) != nullptr;
}

}  // namespace

ProfScope::ProfScope(const char* name, hipStream_t s) : name_(name), s_(s) {
  if (!g_on.load(std::memory_order_relaxed) || !matches(name)) return;
  if (hipEventCreate(&a_) != hipSuccess) return;
  if (hipEventCreate(&b_) != hipSuccess) {
    (void)hipEventDestroy(a_);
    return;
  }
  if (hipEventRecord(a_, s_) != hipSuccess) {
    (void)hipEventDestroy(a_);
    (void)hipEventDestroy(b_);
    return;
  }
  on_ = true;
}

ProfScope::~ProfScope() {
  if (!on_) return;
  (void)hipEventRecord(b_, s_);
  std::lock_guard<std::mutex> lk(g_mu);
  g_recs.push_back(Rec{name_, a_, b_});
}

}  // namespace gs

using namespace gs;

extern "C" {

int gs_profile_enable(const char* filter) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_filter = filter ? filter : "";
  }
  g_on.store(1);
  return GS_OK;
}

int gs_profile_disable(void) {
  g_on.store(0);
  return GS_OK;
}

int gs_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (Rec& r : g_recs) {
    (void)hipEventSynchronize(r.b);
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_recs.clear();
  return GS_OK;
}

int gs_profile_query(const char* kernel, int64_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return GS_E_INVALID;
  std::lock_guard<std::mutex> lk(g_mu);
  int64_t n = 0;
  double ms = 0.0;
  for (const Rec& r : g_recs) {
    if (std::strcmp(r.name, kernel) != 0) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return GS_E_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return GS_E_HIP;
    ++n;
    ms += t;
  }
  *launches = n;
  *total_ms = ms;
  return GS_OK;
}

}  // extern "C"
