// Side streams for work that overlaps the caller's stream, the graph-capture
// stream, and the per-device dynamic-LDS limits of the library's kernels.
//
// One non-blocking stream (default priority) and two timing-free events per
// host thread and device, created on first use and kept until the process
// ends, with the device's CU count.  Each call forks from the caller's stream with `fork` and joins back
// with `join`, so the caller's stream keeps the library's ordering contract:
// everything a call enqueues runs after earlier work on that stream and before
// later work on it.  Per-thread resources keep calls from different host
// threads from sharing the events.

#include <mutex>
#include <utility>
#include <vector>

#include "moe_launch.h"

namespace moe {

hipError_t side_stream(SideStream* out, int which) {
  thread_local std::vector<SideStream> per_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (which < 0 || which >= kSideStreams) return hipErrorInvalidValue;
  if ((int)per_device.size() <= dev * kSideStreams + which) per_device.resize((dev + 1) * kSideStreams);
  SideStream& s = per_device[dev * kSideStreams + which];
  if (!s.stream) {
    SideStream n{};
    if ((e = hipStreamCreateWithFlags(&n.stream, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&n.cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    s = n;
  }
  *out = s;
  return hipSuccess;
}

// A private non-blocking stream per host thread and device, on which graphs
// are captured (a capture must start on a stream that is not the legacy
// default stream, and capturing on a private one leaves the caller's stream
// free).
hipError_t capture_stream(hipStream_t* out) {
  thread_local std::vector<hipStream_t> per_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((int)per_device.size() <= dev) per_device.resize(dev + 1, nullptr);
  if (!per_device[dev] && (e = hipStreamCreateWithFlags(&per_device[dev], hipStreamNonBlocking)) != hipSuccess)
    return e;
  *out = per_device[dev];
  return hipSuccess;
}

// (kernel, device) pairs whose limit is raised, in a fixed table so that no
// call allocates host memory either; past its capacity the attribute is
// simply set again on every launch (correct, only slower).
hipError_t ensure_dynamic_lds(const void* kernel, int bytes) {
  constexpr int kCap = 512;
  static std::mutex mu;
  static std::pair<const void*, int> done[kCap];
  static int n_done = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n_done; ++i)
    if (done[i].first == kernel && done[i].second == dev) return hipSuccess;
  if ((e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)) != hipSuccess) return e;
  if (n_done < kCap) done[n_done++] = {kernel, dev};
  return hipSuccess;
}

}  // namespace moe
