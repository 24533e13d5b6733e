// Opt-in per-kernel timing: when enabled, every kernel the library launches is
// bracketed by two HIP events recorded on the launch's own stream.  Reading
// the timings waits on those events and accumulates milliseconds per kernel
// name.  Disabled (the default) it costs one branch per launch.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/nystrom.h"
#include "nys_internal.hpp"

namespace nys {
namespace {

struct Rec {
  const char* name;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::vector<Rec> g_pending;
std::vector<hipEvent_t> g_pool;
struct Acc {
  double ms = 0.0;
  long long launches = 0;
};
std::map<std::string, Acc> g_acc;
std::vector<std::string> g_names;  // storage behind the returned name pointers

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

KernelTimer::KernelTimer(const char* name, hipStream_t s) : name_(name), s_(s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  start_ = take_event();
  if (start_) hipEventRecord(start_, s_);
}

KernelTimer::~KernelTimer() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t stop = take_event();
  if (!stop) {
    g_pool.push_back(start_);
    return;
  }
  hipEventRecord(stop, s_);
  g_pending.push_back(Rec{name_, start_, stop});
}

}  // namespace nys

extern "C" {

int nystrom_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(nys::g_mu);
  const int prev = nys::g_on ? 1 : 0;
  nys::g_on = on != 0;
  return prev;
}

int nystrom_timing_read(int max_entries, const char** names, double* total_ms, long long* launches) {
  std::lock_guard<std::mutex> lk(nys::g_mu);
  for (auto& r : nys::g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(r.stop) == hipSuccess && hipEventElapsedTime(&ms, r.start, r.stop) == hipSuccess) {
      auto& a = nys::g_acc[r.name];
      a.ms += ms;
      a.launches += 1;
    }
    nys::g_pool.push_back(r.start);
    nys::g_pool.push_back(r.stop);
  }
  nys::g_pending.clear();
  nys::g_names.clear();
  int count = 0;
  for (auto& kv : nys::g_acc) {
    if (count < max_entries && names && total_ms && launches) {
      nys::g_names.push_back(kv.first);
      total_ms[count] = kv.second.ms;
      launches[count] = kv.second.launches;
    }
    ++count;
  }
  if (names && total_ms && launches)
    for (int i = 0; i < (int)nys::g_names.size(); ++i) names[i] = nys::g_names[i].c_str();
  nys::g_acc.clear();
  return count;
}

}  // extern "C"
