// Combine: the weighted sum of each token's expert outputs plus the shared
// expert's output (Perplexity, "Lower latency and higher throughput with
// multi-node DeepSeek deployment", section "Expert parallelism").
//
// y[t] = y_shared[t] + sum_j w[t,j] * y_sorted[pair_slot[t*k + j]], fp32
// accumulation in the fixed order shared, j = 0..k-1.  Inputs and output are
// in the activation dtype.  One workgroup per token; each thread owns 4
// consecutive hidden columns.

#include "moe_common.h"
#include "moe_launch.h"

namespace {

template <int DT>
__device__ __forceinline__ f32x4 load4(const void* base, size_t idx) {
  if constexpr (DT == MOE_BF16) {
    const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + idx);
    return f32x4{bf16_to_f32((uint16_t)v.x), bf16_to_f32((uint16_t)(v.x >> 16)), bf16_to_f32((uint16_t)v.y),
                 bf16_to_f32((uint16_t)(v.y >> 16))};
  } else {
    return *reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
  }
}

template <int OUT_DT>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y_sorted,
                                                      const void* __restrict__ y_shared,
                                                      const int32_t* __restrict__ pair_slot,
                                                      const float* __restrict__ topk_w, int H, int k,
                                                      void* __restrict__ y) {
  const int t = blockIdx.x;
  __shared__ int slot[64];
  __shared__ float wt[64];
  if (threadIdx.x < k) {
    slot[threadIdx.x] = pair_slot[(size_t)t * k + threadIdx.x];
    wt[threadIdx.x] = topk_w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < H; c += blockDim.x * 4) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (y_shared) acc = load4<OUT_DT>(y_shared, (size_t)t * H + c);
    for (int j = 0; j < k; ++j) {
      const f32x4 v = load4<OUT_DT>(y_sorted, (size_t)slot[j] * H + c);
      const float w = wt[j];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(w, v[i], acc[i]);
    }
    if constexpr (OUT_DT == MOE_BF16) {
      uint16_t* o = static_cast<uint16_t*>(y) + (size_t)t * H + c;
      const uint32_t lo = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
      *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<f32x4*>(static_cast<float*>(y) + (size_t)t * H + c) = acc;
    }
  }
}

}  // namespace

namespace moe {

hipError_t launch_combine(const moe_cfg& c, const void* y_sorted, const void* y_shared,
                          const int32_t* pair_slot, const float* topk_w, void* y, hipStream_t st) {
  if (c.act_dtype == MOE_BF16)
    MOE_LAUNCH("combine", combine_kernel<MOE_BF16>, dim3(c.T), dim3(256), 0, st, y_sorted, y_shared, pair_slot, topk_w,
                       c.H, c.k, y);
  else
    MOE_LAUNCH("combine", combine_kernel<MOE_F32>, dim3(c.T), dim3(256), 0, st, y_sorted, y_shared, pair_slot, topk_w,
                       c.H, c.k, y);
  return hipGetLastError();
}

}  // namespace moe
