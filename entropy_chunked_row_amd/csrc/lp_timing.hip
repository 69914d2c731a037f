// Optional per-kernel timing: when enabled, every library launch is bracketed
// by two HIP events recorded on the launch stream; lp_timing_read() waits for
// them and reports launches and total milliseconds per kernel name.  Off by
// default; when off the launch path does nothing extra.
#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/lp.h"
#include "lp_internal.hpp"

namespace lp {
namespace {

struct Rec {
  const char* name;
  hipEvent_t a, b;
};

std::mutex g_mu;
bool g_on = false;
bool g_clocks = false;
std::vector<Rec> g_recs;
std::vector<hipEvent_t> g_pool;

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

TimedLaunch::TimedLaunch(const char* name, hipStream_t s) : name_(name), s_(s), a_(nullptr) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  a_ = take_event();
  if (a_ && hipEventRecord(a_, s) != hipSuccess) {
    g_pool.push_back(a_);
    a_ = nullptr;
  }
}

TimedLaunch::~TimedLaunch() {
  if (!a_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t b = take_event();
  if (b && hipEventRecord(b, s_) == hipSuccess) {
    g_recs.push_back(Rec{name_, a_, b});
  } else {
    g_pool.push_back(a_);
    if (b) g_pool.push_back(b);
  }
}

bool timing_clocks_on() {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_clocks;
}

}  // namespace lp

extern "C" {

void lp_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(lp::g_mu);
  lp::g_on = on != 0;
  lp::g_clocks = on == 2;
  for (auto& r : lp::g_recs) {
    lp::g_pool.push_back(r.a);
    lp::g_pool.push_back(r.b);
  }
  lp::g_recs.clear();
}

lp_status lp_timing_read(const char* kernel, int64_t* launches, double* total_ms) {
  if (!kernel || !launches || !total_ms) return LP_ERR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lk(lp::g_mu);
  int64_t n = 0;
  double ms = 0.0;
  for (auto& r : lp::g_recs) {
    if (strcmp(r.name, kernel) != 0) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return LP_ERR_HIP;
    float t = 0.f;
    if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) return LP_ERR_HIP;
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return LP_OK;
}

}  // extern "C"

extern "C" lp_status lp_timing_clock(const char* kernel, double* mhz, int64_t* samples) {
  if (!kernel || !mhz || !samples) return LP_ERR_INVALID_ARGUMENT;
  if (strcmp(kernel, "k_fwd_tile") != 0) return LP_ERR_UNSUPPORTED;
  *mhz = 0.0;
  *samples = 0;
  if (hipDeviceSynchronize() != hipSuccess) return LP_ERR_HIP;
  int dev = 0, wall_khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || wall_khz <= 0)
    return LP_ERR_HIP;
  std::vector<unsigned long long> pairs(2 * 65536);
  int64_t n = static_cast<int64_t>(pairs.size() / 2);
  if (lp::read_fwd_clocks(pairs.data(), &n) != hipSuccess) return LP_ERR_HIP;
  double sum = 0.0;
  int64_t used = 0;
  for (int64_t b = 0; b < n; ++b) {
    const unsigned long long dt = pairs[2 * b], dr = pairs[2 * b + 1];
    if (dr == 0) continue;
    sum += static_cast<double>(dt) / static_cast<double>(dr);
    ++used;
  }
  if (used) *mhz = sum / static_cast<double>(used) * wall_khz / 1e3;
  *samples = used;
  return LP_OK;
}
