// Routing statistics of one batch: per-expert load, load per expert-parallel
// rank, load skew and the expert affinity matrix.
//
// The GRACE-MoE summary in the pages builds an expert affinity matrix from
// activation patterns to group experts (section "Expert Grouping") and sizes
// replication by the load skew rho = W_max / W_mean of the group loads
// (section "Expert Replication").  Here A[i][j] counts the tokens routed to
// both i and j (the diagonal holds the per-expert loads) and the groups are
// n_ranks ranges of E / n_ranks consecutive experts.
//
// All counts are integer additions, so the results do not depend on the
// order in which the atomics land.  Entries of topk_idx outside [0, E) are
// skipped.  The affinity matrix is cleared by a fill kernel (not a memset
// node, so the sequence can be captured into a graph).

#include "moe_common.h"
#include "moe_launch.h"

namespace {

__global__ __launch_bounds__(256) void fill_zero_kernel(int32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0;
}

// One thread per (token, slot a): adds 1 to A[e_a][e_b] for every slot b of
// the token (b = a gives the diagonal).
__global__ __launch_bounds__(256) void affinity_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                                                       int32_t* __restrict__ A) {
  const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
  if (p >= (long long)T * k) return;
  const long long t = p / k;
  const int ea = idx[p];
  if (ea < 0 || ea >= E) return;
  for (int b = 0; b < k; ++b) {
    const int eb = idx[t * k + b];
    if (eb >= 0 && eb < E) atomicAdd(&A[(size_t)ea * E + eb], 1);
  }
}

// E <= 128: each workgroup counts a range of tokens into a private LDS copy
// of the matrix (E*E ints <= 64 KB) and adds its non-zero entries to the
// global one, so the atomics on hot entries mostly stay on chip.
constexpr int kAffLdsMaxE = 128;

__global__ __launch_bounds__(256) void affinity_lds_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                                                           int tokens_per_wg, int32_t* __restrict__ A) {
  extern __shared__ int loc[];
  const int n = E * E;
  for (int i = threadIdx.x; i < n; i += 256) loc[i] = 0;
  __syncthreads();
  const long long t0 = (long long)blockIdx.x * tokens_per_wg;
  const long long t1 = min((long long)T, t0 + tokens_per_wg);
  for (long long p = t0 * k + threadIdx.x; p < t1 * k; p += 256) {
    const long long t = p / k;
    const int ea = idx[p];
    if (ea < 0 || ea >= E) continue;
    for (int b = 0; b < k; ++b) {
      const int eb = idx[t * k + b];
      if (eb >= 0 && eb < E) atomicAdd(&loc[ea * E + eb], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += 256)
    if (loc[i]) atomicAdd(&A[i], loc[i]);
}

// One workgroup: LDS histogram of the pairs, then rank loads and skews.
__global__ __launch_bounds__(1024) void loads_kernel(const int32_t* __restrict__ idx, int P, int E, int n_ranks,
                                                     int32_t* counts, int32_t* rank_load, float* skew) {
  __shared__ int hist[256];
  __shared__ int rload[256];
  const int tid = threadIdx.x;
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += 1024) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  const int per = E / n_ranks;
  if (tid < n_ranks) {
    int s = 0;
    for (int e = tid * per; e < (tid + 1) * per; ++e) s += hist[e];
    rload[tid] = s;
  }
  __syncthreads();
  if (counts && tid < E) counts[tid] = hist[tid];
  if (rank_load && tid < n_ranks) rank_load[tid] = rload[tid];
  if (skew && tid == 0) {
    int mr = 0, me = 0;
    for (int r = 0; r < n_ranks; ++r) mr = max(mr, rload[r]);
    for (int e = 0; e < E; ++e) me = max(me, hist[e]);
    // rho = max load / mean load, the mean being P / (number of groups)
    skew[0] = P ? (float)mr / ((float)P / (float)n_ranks) : 0.f;
    skew[1] = P ? (float)me / ((float)P / (float)E) : 0.f;
  }
}

}  // namespace

namespace moe {

hipError_t launch_routing_stats(const moe_cfg& c, const int32_t* idx, int n_ranks, int32_t* counts,
                                int32_t* rank_load, float* skew, int32_t* affinity, hipStream_t st) {
  const long long P = (long long)c.T * c.k;
  if (counts || rank_load || skew) {
    MOE_LAUNCH("stats_loads", loads_kernel, dim3(1), dim3(1024), 0, st, idx, (int)P, c.E, n_ranks, counts, rank_load,
               skew);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (affinity) {
    const size_t n = (size_t)c.E * c.E;
    MOE_LAUNCH("stats_clear", fill_zero_kernel, dim3((unsigned)ceil_div((long long)n, 256LL)), dim3(256), 0, st,
               affinity, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (c.E <= kAffLdsMaxE) {
      const int wgs = ceil_div(c.T, 64) < 512 ? ceil_div(c.T, 64) : 512;    // >= 64 tokens per workgroup
      const int per = ceil_div(c.T, wgs);
      MOE_LAUNCH("stats_affinity", affinity_lds_kernel, dim3(wgs), dim3(256), (size_t)c.E * c.E * sizeof(int), st,
                 idx, c.T, c.k, c.E, per, affinity);
    } else {
      MOE_LAUNCH("stats_affinity", affinity_kernel, dim3((unsigned)ceil_div(P, 256LL)), dim3(256), 0, st, idx, c.T,
                 c.k, c.E, affinity);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace moe
