// Per-row 1 x block quantisation to OCP FP8 E4M3.
//
// Perplexity's "Lower latency and higher throughput with multi-node DeepSeek
// deployment" (section "Quantization") quantises activations on the fly with
// one scale per 128-element vector, and its SiLU kernel takes each 128-block's
// absolute maximum with a cross-lane reduction.  Here one wave owns one block
// of up to 256 elements (block <= 256): it loads the block, reduces |v| to the
// block maximum with lane shuffles, and writes codes and the fp32 scale.
// scale = amax / 448 (IEEE fp32 division; 1 for an all-zero block) and
// code = e4m3(v / scale) with round-to-nearest-even and saturation.

#include "moe_common.h"
#include "moe_launch.h"

namespace {

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
  const int grid = (int)((nb + 3) / 4);
  if (grid == 0) return hipSuccess;
  if (in_dtype == MOE_BF16)
    MOE_LAUNCH("quant_fp8", quant_fp8_kernel<MOE_BF16>, dim3(grid), dim3(256), 0, st, in, rows, cols, block, codes, scales);
  else
    MOE_LAUNCH("quant_fp8", quant_fp8_kernel<MOE_F32>, dim3(grid), dim3(256), 0, st, in, rows, cols, block, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
