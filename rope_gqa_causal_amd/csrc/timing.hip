// timing.hip -- per-kernel launch timing for measurement (host code only),
// compiled into the instrumented build (RGC_KERNEL_TIMING) only: the product
// library keeps no global state.
//
// While timing is on, every kernel the library launches is bracketed by two
// HIP events recorded on the stream it is launched on, so each kernel's own
// duration is measured on the device clock, apart from the other kernels of
// the same call.  Events come from a pool that grows on demand and is kept
// for the life of the process; rgc_timing_report waits for the recorded
// events, sums them per kernel and clears the record.  When timing is off a
// launch costs one relaxed atomic load here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"

#ifdef RGC_KERNEL_TIMING
#include "../../include/rgc_timing.h"

namespace rgc {
namespace {

struct Pending {
  const char* name;
  hipEvent_t start, stop;
};
struct Acc {
  long calls = 0;
  double total_ms = 0.0;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
std::map<std::string, Acc> g_acc;

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

KernelTimer::KernelTimer(const char* name, hipStream_t stream) : name_(name), stream_(stream) {
  if (!g_on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(g_mu);
  start_ = take_event();
  stop_ = take_event();
  if (!start_ || !stop_ || hipEventRecord(start_, stream_) != hipSuccess) {
    if (start_) g_pool.push_back(start_);
    if (stop_) g_pool.push_back(stop_);
    start_ = stop_ = nullptr;
  }
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(stop_, stream_) == hipSuccess) {
    g_pending.push_back({name_, start_, stop_});
  } else {
    g_pool.push_back(start_);
    g_pool.push_back(stop_);
  }
}

int timing_enable(int on) {
  g_on.store(on != 0, std::memory_order_relaxed);
  return 0;
}

// Lines "name calls total_us\n"; returns the bytes written (without the
// terminating NUL), or -1 when buf is too small or an event cannot be read.
long timing_report(char* buf, size_t bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  int bad = 0;
  for (const Pending& pe : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(pe.stop) == hipSuccess && hipEventElapsedTime(&ms, pe.start, pe.stop) == hipSuccess) {
      Acc& a = g_acc[pe.name];
      a.calls += 1;
      a.total_ms += ms;
    } else {
      bad = 1;
    }
    g_pool.push_back(pe.start);
    g_pool.push_back(pe.stop);
  }
  g_pending.clear();
  std::string out;
  for (const auto& kv : g_acc) {
    char line[256];
    snprintf(line, sizeof line, "%s %ld %.3f\n", kv.first.c_str(), kv.second.calls, kv.second.total_ms * 1e3);
    out += line;
  }
  g_acc.clear();
  if (bad || !buf || out.size() + 1 > bytes) return -1;
  memcpy(buf, out.c_str(), out.size() + 1);
  return (long)out.size();
}

}  // namespace rgc

extern "C" {

int rgc_timing_enable(int on) { return rgc::timing_enable(on); }

long rgc_timing_report(char* buf, size_t buf_bytes) {
  const long n = rgc::timing_report(buf, buf_bytes);
  return n < 0 ? -10L /* RGC_ERR_ARG */ : n;
}

}  // extern "C"

#endif  // RGC_KERNEL_TIMING
