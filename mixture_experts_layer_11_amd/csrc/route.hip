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

struct RouteOut {
  const float* bias;   // [E] or nullptr
  int32_t* idx;        // [T, k]
  float* w;            // [T, k]
  int E, k, score;
  float rscale;
  int n_group, topk_group;   // group-limited routing; n_group = 1: plain top-k
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
  float kv[4];                                    // selection keys score + bias (-inf past E)
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    const float b = (o.bias && valid[c]) ? o.bias[e] : 0.f;
    kv[c] = valid[c] ? sc[c] + b : -INFINITY;
    key[c] = valid[c] ? (((uint64_t)f32_order_key(kv[c]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e)) : 0ull;
  }
  if (o.n_group > 1 && o.topk_group < o.n_group) {
    // Group-limited routing: lane g < n_group scores group g (experts
    // g*gs .. g*gs+gs-1) by the sum of its two largest keys, gathered with
    // shuffles; topk_group rounds of a wave arg-max pick the groups (ties to
    // the lower group); experts of other groups drop out of the top-k.
    const int gs = o.E / o.n_group;
    const int gl = lane < o.n_group ? lane : o.n_group - 1;
    float b1 = -INFINITY, b2 = -INFINITY;
    for (int i = 0; i < gs; ++i) {
      const int e = gl * gs + i;
      const int src = e & 63, slot = e >> 6;
      const float v0 = __shfl(kv[0], src, 64), v1 = __shfl(kv[1], src, 64);
      const float v2 = __shfl(kv[2], src, 64), v3 = __shfl(kv[3], src, 64);
      const float v = slot == 0 ? v0 : slot == 1 ? v1 : slot == 2 ? v2 : v3;
      if (v > b1) {
        b2 = b1;
        b1 = v;
      } else if (v > b2) {
        b2 = v;
      }
    }
    uint64_t gkey = lane < o.n_group
                        ? (((uint64_t)f32_order_key(b1 + b2) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)lane))
                        : 0ull;
    uint64_t chosen = 0;                          // bit g: group g stays eligible
    for (int j = 0; j < o.topk_group; ++j) {
      const uint64_t best = wave_max_u64(gkey);
      chosen |= 1ull << (0xFFFFFFFFu - (uint32_t)best);
      if (gkey == best) gkey = 0ull;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (valid[c] && !((chosen >> ((lane + 64 * c) / gs)) & 1ull)) key[c] = 0ull;
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

// Gate GEMM over fragments [f0, f1) of K for a 16-token tile.  The four
// waves split the range four ways; each accumulates all ceil(E/16) expert
// tiles (MAXT >= that count) and the four partials are added in wave order
// through LDS (fixed order: reproducible).
template <int DT, bool FUSED, int MAXT>
__global__ __launch_bounds__(256) void gate_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ wg,
                                                   int T, int H, int nsplit, float* __restrict__ part,
                                                   RouteOut o) {
  using F = Frag<DT>;
  extern __shared__ float red[];                  // [4 waves][16 tokens][ldw]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int t0 = blockIdx.x * kTokTile;
  const int s = blockIdx.y;
  const int nfrag = H / F::KF;
  const int f0 = (int)((long long)nfrag * s / nsplit), f1 = (int)((long long)nfrag * (s + 1) / nsplit);
  const int wf0 = f0 + (int)((long long)(f1 - f0) * wave / 4), wf1 = f0 + (int)((long long)(f1 - f0) * (wave + 1) / 4);
  const int E = o.E;
  const int ntiles = (E + 15) >> 4;
  const int ldw = ntiles * 16 + 4;
  const size_t rowbytes = (size_t)H * F::ESZ;

  const int t = t0 + row;
  const uint8_t* pa = x + (size_t)(t < T ? t : T - 1) * rowbytes + grp * 16;   // rows past T: never stored
  const uint8_t* pb[MAXT];
#pragma unroll
  for (int j = 0; j < MAXT; ++j) {
    const int e = min(j * 16 + row, E - 1);     // experts past E: never selected
    pb[j] = wg + (size_t)e * rowbytes + grp * 16;
  }
  f32x4 acc[MAXT];
#pragma unroll
  for (int j = 0; j < MAXT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int U = MAXT >= 8 ? 1 : (MAXT >= 4 ? 2 : 4);   // fragments per trip: ~8 loads in flight
  int f = wf0;
  for (; f + U <= wf1; f += U) {
    i32x4 av[U], bv[U][MAXT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t off = (size_t)(f + u) * 64;
      av[u] = ld16(pa + off);
#pragma unroll
      for (int j = 0; j < MAXT; ++j)
        if (j < ntiles) bv[u][j] = ld16(pb[j] + off);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < MAXT; ++j)
        if (j < ntiles) F::mma(acc[j], av[u], bv[u][j]);
  }
  for (; f < wf1; ++f) {
    const size_t off = (size_t)f * 64;
    const i32x4 av = ld16(pa + off);
#pragma unroll
    for (int j = 0; j < MAXT; ++j)
      if (j < ntiles) F::mma(acc[j], av, ld16(pb[j] + off));
  }

  // acc[j][i] = partial logit of token t0 + 4*grp + i, expert 16*j + row
  float* mine = red + (size_t)wave * 16 * ldw;
#pragma unroll
  for (int j = 0; j < MAXT; ++j)
    if (j < ntiles) {
#pragma unroll
      for (int i = 0; i < 4; ++i) mine[(4 * grp + i) * ldw + 16 * j + row] = acc[j][i];
    }
  __syncthreads();
  // sum the four waves in order into wave 0's region
  for (int idx = threadIdx.x; idx < 16 * ntiles * 16; idx += 256) {
    const int r = idx / (ntiles * 16), e = idx % (ntiles * 16);
    float v = red[r * ldw + e];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += red[(size_t)w * 16 * ldw + r * ldw + e];
    red[r * ldw + e] = v;
  }
  __syncthreads();
  if constexpr (FUSED) {
    for (int r = wave * 4; r < wave * 4 + 4; ++r) {
      const int tt = t0 + r;
      if (tt >= T) break;
      float lg[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        lg[c] = e < E ? red[r * ldw + e] : 0.f;
      }
      route_token(lg, tt, o);
    }
  } else {
    for (int idx = threadIdx.x; idx < 16 * E; idx += 256) {
      const int r = idx / E, e = idx % E;
      const int tt = t0 + r;
      if (tt < T) part[((size_t)s * T + tt) * E + e] = red[r * ldw + e];
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

template <int DT, bool FUSED>
static void launch_gate(const moe_cfg& c, dim3 grid, const uint8_t* xb, const uint8_t* wb, int s, float* part,
                        const RouteOut& o, hipStream_t st) {
  const int ntiles = ceil_div(c.E, 16);
  const size_t smem = (size_t)4 * 16 * (ntiles * 16 + 4) * sizeof(float);
  const char* name = FUSED ? "route_gate_fused" : "route_gate_split";
  if (ntiles <= 2)
    MOE_LAUNCH(name, (gate_kernel<DT, FUSED, 2>), grid, dim3(256), smem, st, xb, wb, c.T, c.H, s, part, o);
  else if (ntiles <= 4)
    MOE_LAUNCH(name, (gate_kernel<DT, FUSED, 4>), grid, dim3(256), smem, st, xb, wb, c.T, c.H, s, part, o);
  else if (ntiles <= 8)
    MOE_LAUNCH(name, (gate_kernel<DT, FUSED, 8>), grid, dim3(256), smem, st, xb, wb, c.T, c.H, s, part, o);
  else
    MOE_LAUNCH(name, (gate_kernel<DT, FUSED, 16>), grid, dim3(256), smem, st, xb, wb, c.T, c.H, s, part, o);
}

hipError_t launch_route(const moe_cfg& c, const void* x, const void* wg, const float* bias, int32_t* idx,
                        float* w, float* part, hipStream_t st) {
  RouteOut o{bias, idx, w, c.E, c.k, c.score, c.routed_scale, c.n_group, c.topk_group};
  const int tiles = ceil_div(c.T, kTokTile);
  const int s = route_splits(c);
  dim3 grid(tiles, s);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  const uint8_t* wb = static_cast<const uint8_t*>(wg);
  if (s == 1) {
    if (c.act_dtype == MOE_F32)
      launch_gate<MOE_F32, true>(c, grid, xb, wb, 1, nullptr, o, st);
    else
      launch_gate<MOE_BF16, true>(c, grid, xb, wb, 1, nullptr, o, st);
    return hipGetLastError();
  }
  if (c.act_dtype == MOE_F32)
    launch_gate<MOE_F32, false>(c, grid, xb, wb, s, part, o, st);
  else
    launch_gate<MOE_BF16, false>(c, grid, xb, wb, s, part, o, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  MOE_LAUNCH("route_reduce_select", route_reduce_kernel, dim3(c.T), dim3(256), 0, st, part, c.T, s, o);
  return hipGetLastError();
}

}  // namespace moe
