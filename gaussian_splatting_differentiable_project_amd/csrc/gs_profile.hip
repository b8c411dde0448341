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

// ---- fp32 VALU throughput probe (measurement helper) ----
// Each lane runs eight independent dependency chains of one instruction
// kind, so the loop issues back to back and its rate is the issue rate of
// that instruction: kind 0 a plain fp32 FMA (v_fma_f32), kind 1 the
// hardware base-2 exponential (v_exp_f32). The chains' sums are written out
// so nothing is dead.
namespace gs {
namespace {

template <int KIND>
__global__ __launch_bounds__(256) void k_valu_probe(int iters, float seed, float b, float c,
                                                    float* __restrict__ out) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = seed + 1e-7f * float(threadIdx.x) + 0.01f * float(i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if constexpr (KIND == 0)
        a[i] = fmaf(a[i], b, c);
      else
        a[i] = __builtin_amdgcn_exp2f(-a[i]);  // stays in (0.5, 1)
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += a[i];
  out[int64_t(blockIdx.x) * 256 + threadIdx.x] = s;
}

}  // namespace
}  // namespace gs

extern "C" int gs_valu_probe(void* stream, int32_t kind, int32_t blocks, int32_t iters,
                             float* out) {
  if (kind < 0 || kind > 1 || blocks < 1 || iters < 1 || !out) return GS_E_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (kind == 0)
    hipLaunchKernelGGL(gs::k_valu_probe<0>, dim3(uint32_t(blocks)), dim3(256), 0, s, iters, 0.5f,
                       0.9999999f, 1e-7f, out);
  else
    hipLaunchKernelGGL(gs::k_valu_probe<1>, dim3(uint32_t(blocks)), dim3(256), 0, s, iters, 0.5f,
                       0.f, 0.f, out);
  return hipGetLastError() == hipSuccess ? GS_OK : GS_E_HIP;
}
