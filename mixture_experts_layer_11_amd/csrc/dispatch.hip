// Dispatch: per-expert aggregation of the routing as an on-device counting sort.
//
// Perplexity's "Lower latency and higher throughput with multi-node DeepSeek
// deployment" (section "MoE router") notes that dense dispatch consumes the
// routing aggregated per expert rather than per token.  Up to 4096 pairs one
// workgroup does it all (dispatch_small_kernel); above, three kernels:
//   1. count:   LDS-atomic histogram of each segment of 256 pairs;
//   2. scan:    per expert, running sum over segments (segment bases and the
//               totals), then an exclusive scan over experts (offsets);
//   3. scatter: one wave per segment walks its pairs in order, 64 at a time;
//               a pair's rank among equal experts of lower lane comes from a
//               64-step register scan of the wave's expert ids, so the
//               placement is stable (ascending pair id inside each expert).
// Integer atomics only feed the histogram, so the result is deterministic.
// Expert ids outside [0, E) are skipped: counted nowhere, never used as an
// address, and their pairs get pair_slot = -1.

#include "moe_common.h"
#include "moe_launch.h"
#include "plan.h"

namespace {

constexpr int kSeg = moe::kDispatchSeg;

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                             int32_t* __restrict__ seg_counts) {
  __shared__ int hist[256];
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int p = blockIdx.x * kSeg + threadIdx.x;
  if (p < P) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) seg_counts[(size_t)blockIdx.x * E + e] = hist[e];
}

// TPE threads per expert (1024 / TPE experts per pass) each own a contiguous
// run of segments: they total it (8 loads in flight), the runs' totals are
// scanned in LDS, then each thread writes its segments' bases.
template <bool PLAN>
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(const int32_t* __restrict__ seg_counts, int nseg,
                                                             int E, int tpe, int32_t* __restrict__ seg_base,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets, moe::PlanArgs pa) {
  __shared__ int part[1024];
  __shared__ int tot[256];
  const int e = threadIdx.x / tpe;     // expert of this thread (E * tpe <= 1024)
  const int q = threadIdx.x % tpe;     // its run of segments
  const int s0 = (int)((long long)nseg * q / tpe), s1 = (int)((long long)nseg * (q + 1) / tpe);
  int run = 0;
  if (e < E) {
    int s = s0;
    for (; s + 8 <= s1; s += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = seg_counts[(size_t)(s + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) run += v[u];
    }
    for (; s < s1; ++s) run += seg_counts[(size_t)s * E + e];
  }
  part[threadIdx.x] = run;
  __syncthreads();
  if (q == 0 && e < E) {                 // per-expert exclusive scan over its runs, in run order
    int acc = 0;
    for (int r = 0; r < tpe; ++r) {
      const int v = part[e * tpe + r];
      part[e * tpe + r] = acc;
      acc += v;
    }
    counts[e] = acc;
    tot[e] = acc;
  }
  __syncthreads();
  if (e < E) {
    int b = part[threadIdx.x];
    int s = s0;
    for (; s + 8 <= s1; s += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = seg_counts[(size_t)(s + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        seg_base[(size_t)(s + u) * E + e] = b;
        b += v[u];
      }
    }
    for (; s < s1; ++s) {
      seg_base[(size_t)s * E + e] = b;
      b += seg_counts[(size_t)s * E + e];
    }
  }
  // exclusive scan of the expert totals (E <= 256) by the first 256 threads
  if (threadIdx.x < 256 && threadIdx.x >= E) tot[threadIdx.x] = 0;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    int v = 0;
    if (threadIdx.x < 256 && threadIdx.x >= d) v = tot[threadIdx.x - d];
    __syncthreads();
    if (threadIdx.x < 256) tot[threadIdx.x] += v;
    __syncthreads();
  }
  if (threadIdx.x < E) offsets[threadIdx.x] = threadIdx.x == 0 ? 0 : tot[threadIdx.x - 1];
  if (threadIdx.x == 0) offsets[E] = tot[E - 1];
  if constexpr (PLAN) {   // the FFN's work lists from the totals (tot[] now holds their inclusive scan)
    __shared__ int wt[moe::ffn::kPlanLds];
    const int g = threadIdx.x;
    int m = 0;   // group g's rows: expert g's total, or all T tokens for the shared expert
    if (g < E) m = tot[g] - (g == 0 ? 0 : tot[g - 1]);
    else if (g < pa.G) m = pa.T;
    moe::ffn::build_plan(pa, m, wt);
  }
}

__global__ __launch_bounds__(64) void dispatch_scatter_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ seg_base,
                                                              int32_t* __restrict__ sorted_pair,
                                                              int32_t* __restrict__ pair_slot) {
  __shared__ int run[256];
  const int lane = threadIdx.x;
  const int s = blockIdx.x;
  for (int e = lane; e < E; e += 64) run[e] = offsets[e] + seg_base[(size_t)s * E + e];
  __syncthreads();
  for (int c = 0; c < kSeg; c += 64) {
    const int p = s * kSeg + c + lane;
    int e = p < P ? idx[p] : -1;
    if (e < 0 || e >= E) e = -1;
    int rank = 0, same = 0;
    for (int j = 0; j < 64; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j);
      const int eq = (ej == e) ? 1 : 0;
      same += eq;
      rank += (j < lane) ? eq : 0;
    }
    if (e >= 0) {
      const int slot = run[e] + rank;
      sorted_pair[slot] = p;
      pair_slot[p] = slot;
    } else if (p < P) {
      pair_slot[p] = -1;                 // skipped id: the combine adds nothing for it
    }
    __syncthreads();
    if (e >= 0 && rank == same - 1) run[e] += same;
    __syncthreads();
  }
}

// Up to kSmallP pairs (decode batches): the whole dispatch in one workgroup
// of 16 waves, saving two launches.  LDS histogram -> exclusive scan ->
// pairs in chunks of 1024 in order: a pair's slot is its expert's running
// base, plus the counts of its expert in the chunk's earlier waves, plus its
// rank among equal experts of lower lane (the same 64-step register scan).
constexpr int kSmallP = 4096;

// With PLAN the workgroup then builds the expert FFN's work lists from the
// histogram it holds (the FFN's plan launch is skipped).
template <bool PLAN>
__global__ __launch_bounds__(1024) void dispatch_small_kernel(const int32_t* __restrict__ idx, int P, int E,
                                                              int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_pair,
                                                              int32_t* __restrict__ pair_slot, moe::PlanArgs pa) {
  __shared__ int hist[256];
  __shared__ int run[256];
  __shared__ int wcnt[16][256];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  // exclusive scan of the expert totals by the first 256 threads
  int v = tid < 256 ? hist[tid] : 0;
  if (tid < 256) run[tid] = v;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int u = (tid < 256 && tid >= d) ? run[tid - d] : 0;
    __syncthreads();
    if (tid < 256) run[tid] += u;
    __syncthreads();
  }
  if (tid < E) {
    counts[tid] = v;
    offsets[tid] = run[tid] - v;
  }
  if (tid == 0) offsets[E] = run[E - 1];
  __syncthreads();
  if (tid < 256) run[tid] -= v;                      // running base: exclusive offsets
  for (int c = 0; c < P; c += 1024) {
    for (int i = tid; i < 16 * 256; i += 1024) (&wcnt[0][0])[i] = 0;
    const int p = c + tid;
    int e = p < P ? idx[p] : -1;
    if (e < 0 || e >= E) e = -1;
    int rank = 0, same = 0;
    for (int j = 0; j < 64; ++j) {
      const int ej = __builtin_amdgcn_readlane(e, j);
      const int eq = (ej == e) ? 1 : 0;
      same += eq;
      rank += (j < lane) ? eq : 0;
    }
    __syncthreads();
    if (e >= 0 && rank == same - 1) wcnt[wave][e] = same;   // last occurrence in the wave
    __syncthreads();
    if (e >= 0) {
      int slot = run[e] + rank;
      for (int w = 0; w < wave; ++w) slot += wcnt[w][e];
      sorted_pair[slot] = p;
      pair_slot[p] = slot;
    } else if (p < P) {
      pair_slot[p] = -1;                 // skipped id: the combine adds nothing for it
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
      for (int w = 0; w < 16; ++w) add += wcnt[w][tid];
      run[tid] += add;
    }
    __syncthreads();
  }
  if constexpr (PLAN) {
    __shared__ int wt[moe::ffn::kPlanLds];
    int m = 0;   // group tid's rows: the histogram, or all T tokens for the shared expert
    if (tid < pa.G) m = tid < E ? hist[tid] : pa.T;
    moe::ffn::build_plan(pa, m, wt);
  }
}

}  // namespace

namespace moe {

static int dispatch_nseg(const moe_cfg& c) { return ceil_div((long long)c.T * c.k, kSeg); }

size_t dispatch_ws_bytes(const moe_cfg& c) { return 2 * (size_t)dispatch_nseg(c) * c.E * sizeof(int32_t); }

hipError_t launch_dispatch(const moe_cfg& c, const int32_t* idx, int32_t* counts, int32_t* offsets,
                           int32_t* sorted_pair, int32_t* pair_slot, int32_t* seg_ws, hipStream_t st,
                           const PlanArgs* plan, bool* planned) {
  const int P = c.T * c.k;
  if (planned) *planned = false;
  if (P <= kSmallP) {
    if (plan) {
      MOE_LAUNCH("dispatch_small", dispatch_small_kernel<true>, dim3(1), dim3(1024), 0, st, idx, P, c.E, counts,
                 offsets, sorted_pair, pair_slot, *plan);
    } else {
      MOE_LAUNCH("dispatch_small", dispatch_small_kernel<false>, dim3(1), dim3(1024), 0, st, idx, P, c.E, counts,
                 offsets, sorted_pair, pair_slot, PlanArgs{});
    }
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess && plan && planned) *planned = true;
    return e;
  }
  const int nseg = dispatch_nseg(c);
  int32_t* seg_counts = seg_ws;
  int32_t* seg_base = seg_ws + (size_t)nseg * c.E;
  MOE_LAUNCH("dispatch_count", dispatch_count_kernel, dim3(nseg), dim3(kSeg), 0, st, idx, P, c.E, seg_counts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int tpe = 1;                       // threads per expert in the scan
  while (tpe * 2 * c.E <= 1024 && tpe * 2 <= nseg) tpe *= 2;
  if (plan) {   // the scan holds the per-expert totals: it also builds the FFN plan
    MOE_LAUNCH("dispatch_scan", dispatch_scan_kernel<true>, dim3(1), dim3(1024), 0, st, seg_counts, nseg, c.E, tpe,
               seg_base, counts, offsets, *plan);
  } else {
    MOE_LAUNCH("dispatch_scan", dispatch_scan_kernel<false>, dim3(1), dim3(1024), 0, st, seg_counts, nseg, c.E, tpe,
               seg_base, counts, offsets, PlanArgs{});
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (plan && planned) *planned = true;
  MOE_LAUNCH("dispatch_scatter", dispatch_scatter_kernel, dim3(nseg), dim3(64), 0, st, idx, P, c.E, offsets, seg_base,
                     sorted_pair, pair_slot);
  return hipGetLastError();
}

}  // namespace moe
