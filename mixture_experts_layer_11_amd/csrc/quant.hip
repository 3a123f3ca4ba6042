// Per-row 1 x block quantisation to OCP FP8 E4M3.
//
// Perplexity's "Lower latency and higher throughput with multi-node DeepSeek
// deployment" (section "Quantization") quantises activations on the fly with
// one scale per 128-element vector, and its SiLU kernel takes each 128-block's
// absolute maximum with a cross-lane reduction.  scale = amax / 448 (IEEE
// fp32 division; 1 for an all-zero block) and code = e4m3(v / scale) with
// round-to-nearest-even and saturation.
//
// Blocks of 64, 128 or 256 elements: the blocks tile the row-major matrix,
// so block b is elements [b * block, (b + 1) * block) of the flat array.  A
// lane takes 8 consecutive elements (one or two 16-byte loads, one 8-byte
// store of codes) and block / 8 lanes of one wave share a block, reducing
// |v| with lane shuffles; the whole matrix streams through at full width.
// Blocks of 192: one wave per block (the general kernel).

#include "moe_common.h"
#include "moe_launch.h"

namespace {

template <int IN_DT, int LPB>
__global__ __launch_bounds__(256) void quant_fp8_vec_kernel(const void* __restrict__ in, long long n8,
                                                            uint8_t* __restrict__ codes, float* __restrict__ scales) {
  static_assert(LPB == 8 || LPB == 16 || LPB == 32, "block / 8 lanes per block");
  const long long gi = (long long)blockIdx.x * 256 + threadIdx.x;   // this lane's group of 8 elements
  const bool valid = gi < n8;   // whole blocks are valid or not, so a shuffle group agrees
  float v[8];
  if (valid) {
    if constexpr (IN_DT == MOE_BF16) {
      const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(in) + gi * 8);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_to_f32((uint16_t)(w[i] & 0xFFFFu));
        v[2 * i + 1] = bf16_to_f32((uint16_t)(w[i] >> 16));
      }
    } else {
      const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(in) + gi * 8);
      const float4 lo = p[0], hi = p[1];
      v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
      v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
  for (int o = LPB / 2; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (!valid) return;
  const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    lo |= f32_to_e4m3(v[i] / scale) << (8 * i);
    hi |= f32_to_e4m3(v[4 + i] / scale) << (8 * i);
  }
  *reinterpret_cast<uint2*>(codes + gi * 8) = make_uint2(lo, hi);
  if ((threadIdx.x & (LPB - 1)) == 0) scales[gi / LPB] = scale;
}

template <int IN_DT>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const void* __restrict__ in, int rows, int cols, int block,
                                                        uint8_t* __restrict__ codes, float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const long long nb = (long long)rows * (cols / block);
  const long long b = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= nb) return;
  const int per_row = cols / block;
  const long long r = b / per_row;
  const int c0 = (int)(b % per_row) * block;
  const size_t base = (size_t)r * cols + c0;
  float v[4];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    float x = 0.f;
    if (c < block) {
      if constexpr (IN_DT == MOE_BF16)
        x = bf16_to_f32(static_cast<const uint16_t*>(in)[base + c]);
      else
        x = static_cast<const float*>(in)[base + c];
    }
    v[i] = x;
    amax = fmaxf(amax, fabsf(x));
  }
  amax = wave_max_f32(amax);
  const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane + 64 * i;
    if (c < block) codes[base + c] = (uint8_t)f32_to_e4m3(v[i] / scale);
  }
  if (lane == 0) scales[(size_t)r * per_row + c0 / block] = scale;
}

}  // namespace

namespace moe {

hipError_t launch_quant_fp8(int rows, int cols, int block, const void* in, int in_dtype, uint8_t* codes,
                            float* scales, hipStream_t st) {
  const long long nb = (long long)rows * (cols / block);
  if (nb == 0) return hipSuccess;
  if (block == 64 || block == 128 || block == 256) {
    const long long n8 = nb * (block / 8);
    const dim3 grid((unsigned)((n8 + 255) / 256));
#define MOE_QV(DT, L) MOE_LAUNCH("quant_fp8", (quant_fp8_vec_kernel<DT, L>), grid, dim3(256), 0, st, in, n8, codes, scales)
    if (in_dtype == MOE_BF16) {
      if (block == 64) MOE_QV(MOE_BF16, 8); else if (block == 128) MOE_QV(MOE_BF16, 16); else MOE_QV(MOE_BF16, 32);
    } else {
      if (block == 64) MOE_QV(MOE_F32, 8); else if (block == 128) MOE_QV(MOE_F32, 16); else MOE_QV(MOE_F32, 32);
    }
#undef MOE_QV
    return hipGetLastError();
  }
  const int grid = (int)((nb + 3) / 4);
  if (in_dtype == MOE_BF16)
    MOE_LAUNCH("quant_fp8", quant_fp8_kernel<MOE_BF16>, dim3(grid), dim3(256), 0, st, in, rows, cols, block, codes, scales);
  else
    MOE_LAUNCH("quant_fp8", quant_fp8_kernel<MOE_F32>, dim3(grid), dim3(256), 0, st, in, rows, cols, block, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
