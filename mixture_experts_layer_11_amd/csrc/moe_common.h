// Internal device helpers of the MI355X MoE library (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

#define MOE_WAVE 64

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ scalar conversions

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Order-preserving map of an fp32 key to uint32 (larger float -> larger uint).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// OCP E4M3 encode of an fp32 value: round to nearest even on the 3-bit
// mantissa, subnormals below 2^-6 (step 2^-9), saturation at +-448.
// Works on the fp32 bit pattern; the sign is kept for values rounding to 0.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;            // |v| >= 448 (no NaN inputs)
  if (a < 0x3C800000u) {                                 // |v| < 2^-6: subnormal grid 2^-9
    // q = rne(|v| * 2^9); |v|*2^9 < 8 is exact in fp32.
    float s = __uint_as_float(a) * 512.0f;
    float r = __builtin_rintf(s);                        // ties to even
    return sign | (uint32_t)r;                           // r == 8 gives 0x08, the smallest normal
  }
  // normal: keep 3 mantissa bits, round to nearest even on the dropped 20 bits
  uint32_t rounded = a + 0x7FFFFu + ((a >> 20) & 1u);
  uint32_t e = (rounded >> 23) - 127 + 7;                // biased e4m3 exponent, >= 1
  uint32_t m = (rounded >> 20) & 7u;
  uint32_t code = (e << 3) | m;
  if (code > 0x7Eu) code = 0x7Eu;                        // rounding up past 448
  return sign | code;
}

// ------------------------------------------------------------------ wave reductions

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ------------------------------------------------------------------ MFMA fragments
//
// A "fragment" is 16 bytes per lane of one operand of a 16x16 MFMA tile:
// lane l holds row (l % 16) of A (or column (l % 16) of B) and the 16-byte
// run of K starting at element (l / 16) * EPL inside the fragment's K window
// of KF = 4 * EPL elements.  Because the A and B fragments assign the same
// K indices to the same (lane group, register slot), any consistent
// assignment computes the same dot products; the C tile comes back with
// lane l holding rows 4*(l/16)+i, i = 0..3, of column l % 16.

template <int DT> struct Frag;

template <> struct Frag<MOE_F32> {
  static constexpr int ESZ = 4, EPL = 4, KF = 16;
  __device__ static __forceinline__ void mma(f32x4& acc, const i32x4& a, const i32x4& b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__int_as_float(a[j]), __int_as_float(b[j]), acc, 0, 0, 0);
  }
};

template <> struct Frag<MOE_BF16> {
  static constexpr int ESZ = 2, EPL = 8, KF = 32;
  __device__ static __forceinline__ void mma(f32x4& acc, const i32x4& a, const i32x4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
  }
};

// FP8 E4M3: two fragments (32 bytes per lane, 128 K values) form one
// v_mfma 16x16x128 with unit (2^0) block exponents.
template <> struct Frag<MOE_FP8_E4M3> {
  static constexpr int ESZ = 1, EPL = 16, KF = 64;
  __device__ static __forceinline__ f32x4 mma128(const i32x4& a0, const i32x4& a1, const i32x4& b0,
                                                 const i32x4& b1) {
    i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    i32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
  }
};

__device__ __forceinline__ i32x4 ld16(const void* p) { return *reinterpret_cast<const i32x4*>(p); }
__device__ __forceinline__ i32x4 zero16() { i32x4 z = {0, 0, 0, 0}; return z; }

__device__ __forceinline__ float silu(float g) { return g / (1.0f + expf(-g)); }

// SiLU on the hardware exp2 and reciprocal (about 1 ulp each, a few
// instructions instead of ~25 for the IEEE expf and division), for outputs
// rounded to bf16 or E4M3 afterwards: its error is some 10^-7 relative
// against the 2^-9 or 2^-4 of the rounding (and against the ~10^-5 with
// which the fp8 matrix instructions sum g and u).  Saturates like silu:
// g -> -inf gives -0, +inf gives g.
__device__ __forceinline__ float silu_fast(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.44269504088896341f * g));
}

// The SwiGLU activation for weights of dtype DT: the fast form where h is
// rounded to bf16 or block-quantised to E4M3 next, the IEEE one where h
// stays fp32 (the fp32 layer).
template <int DT>
__device__ __forceinline__ float silu_for(float g) {
  if constexpr (DT == MOE_F32) return silu(g);
  else return silu_fast(g);
}

// ------------------------------------------------------------------ host-side launch helpers

namespace moe {

struct Status {
  int code;
  const char* what;
};

void set_error(const char* fmt, ...);

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace moe
