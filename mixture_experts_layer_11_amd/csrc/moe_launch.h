// Host-side launch functions of the individual stages (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// Brackets one kernel launch with HIP events while moe_profile_start() is on.
class ProfScope {
 public:
  ProfScope(const char* name, hipStream_t stream);
  ~ProfScope();
  ProfScope(const ProfScope&) = delete;
  ProfScope& operator=(const ProfScope&) = delete;

 private:
  const char* name_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

#define MOE_LAUNCH(NAME, KERNEL, GRID, BLOCK, SHMEM, STREAM, ...)            \
  do {                                                                      \
    ::moe::ProfScope moe_prof_scope_((NAME), (STREAM));                     \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHMEM, STREAM, __VA_ARGS__);    \
  } while (0)

// ---- router
int route_splits(const moe_cfg& c);
size_t route_ws_bytes(const moe_cfg& c);
// ctr: the router's counters, kRouteCounters ints at the workspace start,
// zero before a call and zero after it.
constexpr int kRouteCounters = 64;
hipError_t launch_route(const moe_cfg& c, const void* x, const void* wg, const float* bias, int32_t* idx,
                        float* w, float* part, int32_t* ctr, hipStream_t st);

// ---- expert FFN work-list plan inputs besides the per-group row counts, so
// that a kernel already holding the counts (the one-workgroup dispatch) can
// build the plan and spare the FFN its own plan launch
struct PlanArgs {
  int32_t* plan;
  int G, E, T, fat_cap, halves, mid_rest;
  int shared_tiled;   // the shared expert's tiles join the routed tile lists
};
PlanArgs ffn_plan_args(const moe_cfg& c, int32_t* plan);

// ---- dispatch
constexpr int kDispatchSeg = 256;  // pairs per scatter segment (one wave each)
size_t dispatch_ws_bytes(const moe_cfg& c);
// With plan given, the one-workgroup path (up to 4096 pairs) or, above it,
// the scan kernel also builds the FFN plan from the counts and sets *planned.
hipError_t launch_dispatch(const moe_cfg& c, const int32_t* idx, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_pair, int32_t* pair_slot, int32_t* seg_ws, hipStream_t st,
                           const PlanArgs* plan = nullptr, bool* planned = nullptr);

// ---- fp8 block quantisation
hipError_t launch_quant_fp8(int rows, int cols, int block, const void* in, int in_dtype, uint8_t* codes,
                            float* scales, hipStream_t st);

// ---- expert FFN
struct FfnWs {
  int32_t* plan;  // work lists built on the device from the offsets
  void* h;        // SwiGLU output [P + T, I]: bf16 for bf16 weights, fp32 otherwise
  uint8_t* hq;    // fp8: codes of h [P + T, I]
  float* hs;      // fp8: scales of h [P + T, I / qb]
  uint8_t* xq;    // fp8: codes of x [T, H]
  float* xs;      // fp8: scales of x [T, H / qb]
};
size_t ffn_plan_ints(const moe_cfg& c);
size_t ffn_h_elem_bytes(const moe_cfg& c);
// With fork = false every launch stays on st: no side stream is created or
// used (the entry point that allocates nothing).  With down_only the GEMM2
// stage alone runs, on the h already in ws (fp8: its codes and scales, not
// requantised); x is not read and fork is ignored.
hipError_t launch_expert_ffn(const moe_cfg& c, const void* x, const int32_t* offsets,
                             const int32_t* sorted_pair, const moe_weights& w, void* y_sorted,
                             void* y_shared, const FfnWs& ws, hipStream_t st, bool planned = false,
                             bool fork = true, bool down_only = false);

// ---- side stream (streams.cpp): forked from and joined back to the caller's stream
struct SideStream {
  hipStream_t stream;
  hipEvent_t fork;
  hipEvent_t join;
  int cus;          // compute units of the device
};
constexpr int kSideStreams = 2;                   // per host thread and device
// Raises a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per (kernel, device); safe to call from several host threads.
hipError_t ensure_dynamic_lds(const void* kernel, int bytes);
hipError_t side_stream(SideStream* out, int which = 0);
hipError_t capture_stream(hipStream_t* out);   // private stream for graph capture

// ---- routing statistics
hipError_t launch_routing_stats(const moe_cfg& c, const int32_t* idx, int n_ranks, int32_t* counts,
                                int32_t* rank_load, float* skew, int32_t* affinity, hipStream_t st);

// ---- combine
hipError_t launch_combine(const moe_cfg& c, const void* y_sorted, const void* y_shared,
                          const int32_t* pair_slot, const float* topk_w, void* y, hipStream_t st);

}  // namespace moe
