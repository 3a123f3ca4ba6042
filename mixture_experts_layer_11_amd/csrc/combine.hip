// Combine: the weighted sum of each token's expert outputs plus the shared
// expert's output (Perplexity, "Lower latency and higher throughput with
// multi-node DeepSeek deployment", section "Expert parallelism").
//
// y[t] = y_shared[t] + sum_j w[t,j] * y_sorted[pair_slot[t*k + j]], fp32
// accumulation in the fixed order shared, j = 0..k-1; a pair whose slot is
// negative (dispatch skipped its expert id) adds nothing.  Inputs and output
// are in the activation dtype; every row is read once (nontemporal loads).

#include "moe_common.h"
#include "moe_launch.h"

namespace {

// 8 consecutive values of a row as fp32 (16 bytes of bf16, 32 of fp32).
template <int DT>
__device__ __forceinline__ void load8(const void* base, size_t idx, float (&v)[8]) {
  if constexpr (DT == MOE_BF16) {
    const i32x4 q = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(base) + idx));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_to_f32((uint16_t)q[i]);
      v[2 * i + 1] = bf16_to_f32((uint16_t)((uint32_t)q[i] >> 16));
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + idx);
    const f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = a[i];
      v[4 + i] = b[i];
    }
  }
}

// One workgroup per token; each thread owns 8 consecutive hidden columns per
// step (one step when H <= 8192).  KT = k when the launch knows it at compile time (k = 8, the layer's
// top-8), else 0: with a fixed k the k row loads of a step are all issued
// before the first FMA, so a thread keeps k + 1 loads in flight.
// bf16 with k known at compile time (the layer's top-8): the rows stay as
// loaded (8 packed bf16 per 16 bytes) until their multiply-add, half the
// registers of fp32 copies (68 VGPRs against 104), so two 14-wave
// workgroups fit a CU instead of one and twice the rows are in flight
// (prefill8192_ep8: 248 -> 190 us).  Same order of operations, same bits.
template <int KT>
__global__ __launch_bounds__(1024) void combine_bf16_kernel(const void* __restrict__ y_sorted,
                                                           const void* __restrict__ y_shared,
                                                           const int32_t* __restrict__ pair_slot,
                                                           const float* __restrict__ topk_w, int H,
                                                           void* __restrict__ y) {
  const int t = blockIdx.x;
  __shared__ int slot[KT];
  __shared__ float wt[KT];
  if (threadIdx.x < KT) {
    slot[threadIdx.x] = pair_slot[(size_t)t * KT + threadIdx.x];
    wt[threadIdx.x] = topk_w[(size_t)t * KT + threadIdx.x];
  }
  __syncthreads();
  const uint16_t* ys = static_cast<const uint16_t*>(y_sorted);
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    const i32x4 sh = y_shared ? __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(
                                    static_cast<const uint16_t*>(y_shared) + (size_t)t * H + c))
                              : zero16();
    i32x4 v[KT];
#pragma unroll
    for (int j = 0; j < KT; ++j)   // a pair that dispatch skipped (id outside [0, E)) adds nothing
      v[j] = slot[j] >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(ys + (size_t)slot[j] * H + c))
                          : zero16();
    float acc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = bf16_to_f32((uint16_t)sh[i]);
      acc[2 * i + 1] = bf16_to_f32((uint16_t)((uint32_t)sh[i] >> 16));
    }
#pragma unroll
    for (int j = 0; j < KT; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wt[j], bf16_to_f32((uint16_t)v[j][i]), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wt[j], bf16_to_f32((uint16_t)((uint32_t)v[j][i] >> 16)), acc[2 * i + 1]);
      }
    i32x4 q;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      q[i] = (int)((uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16));
    __builtin_nontemporal_store(q, reinterpret_cast<i32x4*>(static_cast<uint16_t*>(y) + (size_t)t * H + c));
  }
}

template <int OUT_DT, int KT>
__global__ __launch_bounds__(1024) void combine_kernel(const void* __restrict__ y_sorted,
                                                      const void* __restrict__ y_shared,
                                                      const int32_t* __restrict__ pair_slot,
                                                      const float* __restrict__ topk_w, int H, int k_rt,
                                                      void* __restrict__ y) {
  const int k = KT > 0 ? KT : k_rt;
  const int t = blockIdx.x;
  __shared__ int slot[64];
  __shared__ float wt[64];
  if (threadIdx.x < k) {
    slot[threadIdx.x] = pair_slot[(size_t)t * k + threadIdx.x];
    wt[threadIdx.x] = topk_w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float acc[8];
    if (y_shared) {
      load8<OUT_DT>(y_shared, (size_t)t * H + c, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    if constexpr (KT > 0) {
      float v[KT][8];
#pragma unroll
      for (int j = 0; j < KT; ++j) {
        if (slot[j] >= 0) {
          load8<OUT_DT>(y_sorted, (size_t)slot[j] * H + c, v[j]);
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
        }
      }
#pragma unroll
      for (int j = 0; j < KT; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wt[j], v[j][i], acc[i]);
    } else {
      for (int j = 0; j < k; ++j) {
        if (slot[j] < 0) continue;     // a pair that dispatch skipped (id outside [0, E))
        float v[8];
        load8<OUT_DT>(y_sorted, (size_t)slot[j] * H + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wt[j], v[i], acc[i]);
      }
    }
    if constexpr (OUT_DT == MOE_BF16) {
      i32x4 q;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        q[i] = (int)((uint32_t)f32_to_bf16(acc[2 * i]) | ((uint32_t)f32_to_bf16(acc[2 * i + 1]) << 16));
      __builtin_nontemporal_store(q, reinterpret_cast<i32x4*>(static_cast<uint16_t*>(y) + (size_t)t * H + c));
    } else {
      f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(y) + (size_t)t * H + c);
      __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, o);
      __builtin_nontemporal_store(f32x4{acc[4], acc[5], acc[6], acc[7]}, o + 1);
    }
  }
}

}  // namespace

namespace moe {

hipError_t launch_combine(const moe_cfg& c, const void* y_sorted, const void* y_shared,
                          const int32_t* pair_slot, const float* topk_w, void* y, hipStream_t st) {
  // one 8-column chunk per thread when a row fits one workgroup (H <= 8192;
  // prefill8192_ep8: 205 -> 194 us against 256 threads looping 3.5 times)
  const int chunks = c.H / 8;
  const int threads = chunks <= 1024 ? (chunks + 63) / 64 * 64 : 1024;
#define MOE_CB(DT, KT)                                                                                             \
  MOE_LAUNCH("combine", (combine_kernel<DT, KT>), dim3(c.T), dim3(threads), 0, st, y_sorted, y_shared, pair_slot, \
             topk_w, c.H, c.k, y)
  if (c.act_dtype == MOE_BF16) {
    if (c.k == 8)
      MOE_LAUNCH("combine", (combine_bf16_kernel<8>), dim3(c.T), dim3(threads), 0, st, y_sorted, y_shared, pair_slot,
                 topk_w, c.H, y);
    else
      MOE_CB(MOE_BF16, 0);
  } else {
    if (c.k == 8) MOE_CB(MOE_F32, 8); else MOE_CB(MOE_F32, 0);
  }
#undef MOE_CB
  return hipGetLastError();
}

}  // namespace moe
