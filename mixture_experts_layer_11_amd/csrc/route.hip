// Router: gate GEMM -> expert scoring -> selection bias -> top-k -> weights.
//
// The four steps are the ones the vLLM DeepSeek-V4.1-Flash article lists for
// its fused router (section "Kernels", item "Mega-Gate"); fusing them saves a
// launch and the round trip of the scores through memory.  Perplexity's
// "Lower latency and higher throughput with multi-node DeepSeek deployment"
// (section "MoE router") describes the selection as a sort that also tracks
// indices; here it is k rounds of a wave-wide arg-max over 64-bit keys
// (order-preserving fp32 key in the high word, complemented expert index in
// the low word, so equal keys go to the lower expert).
//
// Layout: one workgroup (4 waves) owns a tile of 16 tokens and all E <= 256
// experts; wave w accumulates expert tiles w, w+4, w+8, w+12 of 16 experts
// with 16x16 MFMAs.  When the token count is too small to fill the GPU, the
// K range is split over workgroups; each writes fp32 partial logits and a
// second kernel sums them in split order (fixed order: bitwise reproducible)
// before the same epilogue.

#include "moe_common.h"
#include "moe_launch.h"

namespace {

constexpr int kTokTile = 16;
constexpr int kMaxE = 256;
constexpr int kLdsStride = kMaxE + 4;

struct RouteOut {
  const float* bias;   // [E] or nullptr
  int32_t* idx;        // [T, k]
  float* w;            // [T, k]
  int E, k, score;
  float rscale;
};

// Scores, keys, top-k and weights for one token whose logits sit in the
// lanes of one wave: lane l holds experts l, l+64, l+128, l+192.
__device__ void route_token(const float (&lg)[4], int t, const RouteOut& o) {
  const int lane = threadIdx.x & 63;
  float sc[4];
  bool valid[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) valid[c] = lane + 64 * c < o.E;
  if (o.score == MOE_SCORE_SOFTMAX) {
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (valid[c]) m = fmaxf(m, lg[c]);
    m = wave_max_f32(m);
    float ex[4], s = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      ex[c] = valid[c] ? expf(lg[c] - m) : 0.f;
      s += ex[c];
    }
    s = wave_sum_f32(s);
#pragma unroll
    for (int c = 0; c < 4; ++c) sc[c] = ex[c] / s;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) sc[c] = 1.0f / (1.0f + expf(-lg[c]));
  }
  uint64_t key[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    const float b = (o.bias && valid[c]) ? o.bias[e] : 0.f;
    key[c] = valid[c] ? (((uint64_t)f32_order_key(sc[c] + b) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0ull;
  }
  float wsum = 0.f, my_s = 0.f;
  int my_e = 0;
  for (int j = 0; j < o.k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int c = 1; c < 4; ++c) best = key[c] > best ? key[c] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (key[c] == best) key[c] = 0ull;
    const int slot = e >> 6;
    const float mine = slot == 0 ? sc[0] : slot == 1 ? sc[1] : slot == 2 ? sc[2] : sc[3];
    const float s_e = __shfl(mine, e & 63, 64);
    wsum += s_e;
    if (lane == j) {
      my_e = e;
      my_s = s_e;
    }
  }
  if (lane < o.k) {
    o.idx[(size_t)t * o.k + lane] = my_e;
    o.w[(size_t)t * o.k + lane] = my_s / wsum * o.rscale;
  }
}

// Gate GEMM over fragments [f0, f1) of K for a 16-token tile.
template <int DT, bool FUSED>
__global__ __launch_bounds__(256) void gate_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ wg,
                                                   int T, int H, int nsplit, float* __restrict__ part,
                                                   RouteOut o) {
  using F = Frag<DT>;
  __shared__ float lds[FUSED ? kTokTile * kLdsStride : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int t0 = blockIdx.x * kTokTile;
  const int s = blockIdx.y;
  const int nfrag = H / F::KF;
  const int f0 = (int)((long long)nfrag * s / nsplit), f1 = (int)((long long)nfrag * (s + 1) / nsplit);
  const int E = o.E;
  const int ntiles = (E + 15) >> 4;
  const size_t rowbytes = (size_t)H * F::ESZ;

  const int t = t0 + row;
  const bool tval = t < T;
  const uint8_t* pa = x + (size_t)(tval ? t : 0) * rowbytes + grp * 16;
  const uint8_t* pb[4];
  bool ev[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = (wave + 4 * j) * 16 + row;
    ev[j] = e < E;
    pb[j] = wg + (size_t)(ev[j] ? e : 0) * rowbytes + grp * 16;
  }
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 4
  for (int f = f0; f < f1; ++f) {
    const size_t off = (size_t)f * 64;
    const i32x4 a = tval ? ld16(pa + off) : zero16();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (wave + 4 * j < ntiles) {
        const i32x4 b = ev[j] ? ld16(pb[j] + off) : zero16();
        F::mma(acc[j], a, b);
      }
    }
  }

  // acc[j][i] = logit of token t0 + 4*grp + i, expert (wave + 4j)*16 + row
  if constexpr (FUSED) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = (wave + 4 * j) * 16 + row;
      if (wave + 4 * j < ntiles) {
#pragma unroll
        for (int i = 0; i < 4; ++i) lds[(4 * grp + i) * kLdsStride + e] = acc[j][i];
      }
    }
    __syncthreads();
    for (int r = wave * 4; r < wave * 4 + 4; ++r) {
      const int tt = t0 + r;
      if (tt >= T) break;
      float lg[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        lg[c] = e < E ? lds[r * kLdsStride + e] : 0.f;
      }
      route_token(lg, tt, o);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = (wave + 4 * j) * 16 + row;
      if (wave + 4 * j < ntiles && e < E) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tt = t0 + 4 * grp + i;
          if (tt < T) part[((size_t)s * T + tt) * E + e] = acc[j][i];
        }
      }
    }
  }
}

// Sum the split-K partial logits in split order, then select.  One workgroup
// per token: thread e sums expert e's partials (8 independent loads in
// flight, added in split order), wave 0 runs the selection.
__global__ __launch_bounds__(256) void route_reduce_kernel(const float* __restrict__ part, int T, int nsplit,
                                                           RouteOut o) {
  __shared__ float lg_s[kMaxE];
  const int t = blockIdx.x;
  const int e = threadIdx.x;
  if (e < o.E) {
    const float* p = part + (size_t)t * o.E + e;
    const size_t stride = (size_t)T * o.E;
    float v = 0.f;
    int s = 0;
    for (; s + 8 <= nsplit; s += 8) {
      float q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) q[u] = p[(size_t)(s + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) v += q[u];
    }
    for (; s < nsplit; ++s) v += p[(size_t)s * stride];
    lg_s[e] = v;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  float lg[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) lg[c] = lane + 64 * c < o.E ? lg_s[lane + 64 * c] : 0.f;
  route_token(lg, t, o);
}

}  // namespace

namespace moe {

int route_splits(const moe_cfg& c) {
  const int tiles = ceil_div(c.T, kTokTile);
  const int kf = c.act_dtype == MOE_F32 ? Frag<MOE_F32>::KF : Frag<MOE_BF16>::KF;
  const int nfrag = c.H / kf;
  if (tiles >= 256) return 1;
  int s = ceil_div(256, tiles);
  const int smax = nfrag / 8 > 0 ? nfrag / 8 : 1;   // at least 8 fragments of K per split
  return s < smax ? s : smax;
}

size_t route_ws_bytes(const moe_cfg& c) {
  const int s = route_splits(c);
  return s > 1 ? (size_t)s * c.T * c.E * sizeof(float) : 0;
}

hipError_t launch_route(const moe_cfg& c, const void* x, const void* wg, const float* bias, int32_t* idx,
                        float* w, float* part, hipStream_t st) {
  RouteOut o{bias, idx, w, c.E, c.k, c.score, c.routed_scale};
  const int tiles = ceil_div(c.T, kTokTile);
  const int s = route_splits(c);
  dim3 grid(tiles, s), block(256);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const uint8_t* wb = static_cast<const uint8_t*>(wg);
  if (s == 1) {
    if (c.act_dtype == MOE_F32)
      MOE_LAUNCH("route_gate_fused", (gate_kernel<MOE_F32, true>), grid, block, 0, st, xb, wb, c.T, c.H, 1, nullptr, o);
    else
      MOE_LAUNCH("route_gate_fused", (gate_kernel<MOE_BF16, true>), grid, block, 0, st, xb, wb, c.T, c.H, 1, nullptr, o);
    return hipGetLastError();
  }
  if (c.act_dtype == MOE_F32)
    MOE_LAUNCH("route_gate_split", (gate_kernel<MOE_F32, false>), grid, block, 0, st, xb, wb, c.T, c.H, s, part, o);
  else
    MOE_LAUNCH("route_gate_split", (gate_kernel<MOE_BF16, false>), grid, block, 0, st, xb, wb, c.T, c.H, s, part, o);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MOE_LAUNCH("route_reduce_select", route_reduce_kernel, dim3(c.T), block, 0, st, part, c.T, s, o);
  return hipGetLastError();
}

}  // namespace moe
