// Per-kernel launch timing with HIP events (a measurement aid).
//
// While timing is on, every kernel launch of the library is bracketed by a
// pair of HIP events recorded on the launch stream, so the mean duration of
// each kernel can be read back without a profiler. Off (the default), the
// launch sites pay one relaxed load.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>
#include <vector>

#include "lsa.h"
#include "lsa_internal.h"

namespace lsa {

namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Rec> g_recs;         // records since timing was switched on
std::vector<hipEvent_t> g_free;  // events for reuse

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void recycle_all() {
  for (const Rec& r : g_recs) {
    g_free.push_back(r.a);
    g_free.push_back(r.b);
  }
  g_recs.clear();
}

}  // namespace

KernelTimer::KernelTimer(const char* name, hipStream_t st) : name_(name), st_(st), a_(nullptr) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  a_ = take_event();
  if (a_ != nullptr && hipEventRecord((hipEvent_t)a_, st_) != hipSuccess) {
    g_free.push_back((hipEvent_t)a_);
    a_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (a_ == nullptr) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t b = take_event();
  if (b == nullptr || hipEventRecord(b, st_) != hipSuccess) {
    g_free.push_back((hipEvent_t)a_);
    if (b != nullptr) g_free.push_back(b);
    return;
  }
  g_recs.push_back(Rec{name_, (hipEvent_t)a_, b});
}

}  // namespace lsa

extern "C" int32_t lsa_kernel_timing(int32_t on) {
  std::lock_guard<std::mutex> lk(lsa::g_mu);
  // events still pending on a stream are waited for before reuse
  for (const lsa::Rec& r : lsa::g_recs)
    if (hipEventSynchronize(r.b) != hipSuccess) return LSA_HIP;
  lsa::recycle_all();
  lsa::g_on.store(on != 0, std::memory_order_relaxed);
  return LSA_OK;
}

extern "C" int32_t lsa_kernel_time(const char* name, float* ms_mean, int32_t* launches) {
  if (name == nullptr || ms_mean == nullptr || launches == nullptr) return LSA_INVALID_ARG;
  std::lock_guard<std::mutex> lk(lsa::g_mu);
  double sum = 0.0;
  int n = 0;
  for (const lsa::Rec& r : lsa::g_recs) {
    if (std::strcmp(r.name, name) != 0) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return LSA_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return LSA_HIP;
    sum += ms;
    ++n;
  }
  *ms_mean = n > 0 ? (float)(sum / n) : 0.f;
  *launches = n;
  return LSA_OK;
}
