// Per-kernel HIP-event timing (moe_profile_start / moe_profile_stop).

#include <hip/hip_runtime.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "moe_launch.h"

namespace {

struct Mark {
  const char* name;
  hipEvent_t start, stop;
};

std::mutex g_mu;
bool g_on = false;
std::string g_only;   // empty: all kernels
std::vector<Mark> g_marks;
std::vector<hipEvent_t> g_pool;

hipEvent_t get_event() {
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

namespace moe {

ProfScope::ProfScope(const char* name, hipStream_t stream) : name_(name), stream_(stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_on) return;
  if (!g_only.empty() && g_only != name) return;
  start_ = get_event();
  if (start_ && hipEventRecord(start_, stream) != hipSuccess) {
    g_pool.push_back(start_);
    start_ = nullptr;
  }
}

ProfScope::~ProfScope() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  hipEvent_t stop = get_event();
  if (stop && hipEventRecord(stop, stream_) == hipSuccess) {
    g_marks.push_back({name_, start_, stop});
  } else {
    g_pool.push_back(start_);
    if (stop) g_pool.push_back(stop);
  }
}

}  // namespace moe

extern "C" {

int moe_profile_start(const char* only) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = true;
  g_only = only ? only : "";
  return MOE_OK;
}

int moe_profile_stop(moe_kernel_time* out, int32_t max_entries, int32_t* n_entries) {
  std::vector<Mark> marks;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_on = false;
    marks.swap(g_marks);
  }
  std::vector<moe_kernel_time> agg;
  int status = MOE_OK;
  for (const Mark& m : marks) {
    float ms = 0.f;
    if (hipEventSynchronize(m.stop) != hipSuccess || hipEventElapsedTime(&ms, m.start, m.stop) != hipSuccess)
      status = MOE_ERR_HIP;
    size_t i = 0;
    for (; i < agg.size(); ++i)
      if (strncmp(agg[i].name, m.name, sizeof agg[i].name) == 0) break;
    if (i == agg.size()) {
      moe_kernel_time t{};
      strncpy(t.name, m.name, sizeof t.name - 1);
      agg.push_back(t);
    }
    agg[i].launches += 1;
    agg[i].total_ms += ms;
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    for (const Mark& m : marks) {
      g_pool.push_back(m.start);
      g_pool.push_back(m.stop);
    }
  }
  if (n_entries) *n_entries = (int32_t)agg.size();
  if (out)
    for (int32_t i = 0; i < max_entries && i < (int32_t)agg.size(); ++i) out[i] = agg[i];
  return status;
}

}  // extern "C"
