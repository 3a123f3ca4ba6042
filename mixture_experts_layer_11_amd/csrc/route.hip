// Router: gate GEMM -> expert scoring -> selection bias -> top-k -> weights.
//
// The four steps are the ones the vLLM DeepSeek-V4.1-Flash article lists for
// its fused router (section "Kernels", item "Mega-Gate"); fusing them saves a
// launch and the round trip of the scores through memory.  Perplexity's
// "Lower latency and higher throughput with multi-node DeepSeek deployment"
// (section "MoE router") describes the selection as a sort that also tracks
// indices; here it is k rounds of a wave-wide arg-max: the maximum of the
// order-preserving uint32 keys (DPP row reductions), then the lowest expert
// holding it (a ballot), so equal keys go to the lower expert.
//
// Below 512 bf16 tokens (up to 1024 fp32 tokens) the whole router is one
// launch (gate_last_kernel): workgroups split the 16-token tiles' gate GEMM
// by expert groups and K ranges, and the last one to finish a tile sums its
// partials in split order and selects.  From 512 bf16 tokens on, an
// LDS-staged kernel owns 64 or 128 tokens per workgroup, so the gate weights
// are re-read far less often (see gate_tile_kernel); beyond 1024 fp32 tokens
// a workgroup (4 waves) owns a 16-token tile and all E <= 256 experts with
// 16x16 MFMAs straight from global memory (gate_kernel).  When those tiles
// are too few to fill the GPU, the K range is split over workgroups; each
// writes fp32 partial logits and a second kernel sums them in split order
// (fixed order: bitwise reproducible) before the same selection.

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

// Wave-wide maximum of a uint32, returned to every lane: DPP steps reduce
// each row of 16 lanes (lane pairs, quads, half-rows, rows), then the four
// row maxima are read out as scalars.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// Lowest index 64 c + lane whose key[c] equals m (m is the wave maximum, so
// one exists): the ballot of slot 0 covers indices 0..63, slot 1 64..127, ...
__device__ __forceinline__ int lowest_with_key(const uint32_t (&key)[4], uint32_t m) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const uint64_t b = __ballot(key[c] == m);
    if (b) return 64 * c + __builtin_ctzll(b);
  }
  return 0;
}

// Scores, keys, top-k and weights for one token whose logits sit in the
// lanes of one wave: lane l holds experts l, l+64, l+128, l+192.  Selection
// keys are the order-preserving uint32 of score + bias (0: not eligible);
// each of the k rounds takes the wave maximum and, among equal keys, the
// lowest expert.
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
  uint32_t key[4];
  float kv[4];                                    // selection keys score + bias (-inf past E)
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int e = lane + 64 * c;
    const float b = (o.bias && valid[c]) ? o.bias[e] : 0.f;
    kv[c] = valid[c] ? sc[c] + b : -INFINITY;
    key[c] = valid[c] ? f32_order_key(kv[c]) : 0u;   // every finite key maps above 0
  }
  if (o.n_group > 1 && o.topk_group < o.n_group) {
    // Group-limited routing: lane g < n_group scores group g (experts
    // g*gs .. g*gs+gs-1) by the sum of its two largest keys, gathered with
    // shuffles; topk_group rounds of a wave maximum pick the groups (ties to
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
    uint32_t gkey = lane < o.n_group ? f32_order_key(b1 + b2) : 0u;
    uint64_t chosen = 0;                          // bit g: group g stays eligible
    for (int j = 0; j < o.topk_group; ++j) {
      const uint32_t best = wave_max_u32(gkey);
      const int g = __builtin_ctzll(__ballot(gkey == best));
      chosen |= 1ull << g;
      if (lane == g) gkey = 0u;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
      if (valid[c] && !((chosen >> ((lane + 64 * c) / gs)) & 1ull)) key[c] = 0u;
  }
  float wsum = 0.f, my_s = 0.f;
  int my_e = 0;
  for (int j = 0; j < o.k; ++j) {
    const uint32_t m = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
    const int e = lowest_with_key(key, m);
    const int slot = e >> 6, src = e & 63;
    if (lane == src) key[slot] = 0u;
    const float mine = slot == 0 ? sc[0] : slot == 1 ? sc[1] : slot == 2 ? sc[2] : sc[3];
    const float s_e = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine), src));
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

// ---- few tokens: the whole router in one launch
//
// The decode shapes (a few to a few hundred tokens) read the 3.7 MB gate
// weight with little reuse, so the work is spread over many workgroups:
// workgroup (token tile, expert group, K split) computes the partial logits
// of 16 tokens x 64 experts over its K range (8 waves split the range
// further; their partials are added in wave order through LDS) and stores
// them.  It then counts itself done on its token tile's counter; the last
// workgroup to arrive sums the tile's partials over the splits in split order
// (bitwise reproducible) and runs scoring, bias, top-k and weights for the
// tile's 16 tokens, two per wave, and clears the counter for the next call.
// So gate GEMM, scoring, bias and top-k are one launch with no round trip of
// the scores through a second kernel.  Nothing waits on another workgroup:
// each either returns or is the last.  The counters must be zero when a call
// starts; every call leaves them zero.
constexpr int kLastEG = 64;        // experts per workgroup
constexpr int kLastWaves = 8;
constexpr int kLastMaxTiles = 64;  // token tiles (counters) of one call

template <int DT>
__global__ __launch_bounds__(512) void gate_last_kernel(const uint8_t* __restrict__ x, const uint8_t* __restrict__ wg,
                                                        int T, int H, int nsplit, float* __restrict__ part,
                                                        int* __restrict__ ctr, RouteOut o) {
  using F = Frag<DT>;
  __shared__ float red[kLastWaves][16][kLastEG + 4];
  __shared__ float lg_s[16][kMaxE + 4];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int E = o.E;
  const int ng = (E + kLastEG - 1) / kLastEG;
  const int eg = blockIdx.y % ng, s = blockIdx.y / ng;
  const int t0 = blockIdx.x * kTokTile;
  const int e0 = eg * kLastEG;
  const int nt = min(4, (E - e0 + 15) >> 4);          // 16-expert tiles of this group
  const int nfrag = H / F::KF;
  const int f0 = (int)((long long)nfrag * s / nsplit), f1 = (int)((long long)nfrag * (s + 1) / nsplit);
  const int wf0 = f0 + (int)((long long)(f1 - f0) * wave / kLastWaves);
  const int wf1 = f0 + (int)((long long)(f1 - f0) * (wave + 1) / kLastWaves);
  const size_t rowbytes = (size_t)H * F::ESZ;
  const uint8_t* pa = x + (size_t)min(t0 + row, T - 1) * rowbytes + grp * 16;   // rows past T: never stored
  const uint8_t* pb[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) pb[j] = wg + (size_t)min(e0 + j * 16 + row, E - 1) * rowbytes + grp * 16;
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int f = wf0; f < wf1; ++f) {
    const size_t off = (size_t)f * 64;
    const i32x4 av = ld16(pa + off);
    i32x4 bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nt) bv[j] = ld16(pb[j] + off);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < nt) F::mma(acc[j], av, bv[j]);
  }
  // acc[j][i] = partial logit of token t0 + 4 grp + i, expert e0 + 16 j + row
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * grp + i][16 * j + row] = acc[j][i];
  __syncthreads();
  for (int idx = tid; idx < 16 * kLastEG; idx += 512) {
    const int r = idx / kLastEG, e = idx % kLastEG;
    float v = red[0][r][e];
#pragma unroll
    for (int w = 1; w < kLastWaves; ++w) v += red[w][r][e];   // wave order
    // device-scope stores: written through to where every XCD reads them
    if (t0 + r < T && e0 + e < E)
      __hip_atomic_store(&part[((size_t)s * T + t0 + r) * E + e0 + e], v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  // Every thread's stores have completed before the workgroup counts itself
  // done (the barrier waits for them and orders them before the count).  A
  // device-scope release fence would instead write back this XCD's whole L2
  // (512 such fences made the 256-token router 4x slower).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    last = __hip_atomic_fetch_add(&ctr[blockIdx.x], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (int)gridDim.y - 1;
  __syncthreads();
  if (!last) return;
  // logits of the tile's tokens: the partials summed over the splits in split order
  if ((E & 3) == 0) {
    // 16-byte device-scope loads (through a buffer resource, whose cache
    // policy can carry the scope bit), every split's load of two positions
    // issued before the first add
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(part, 0, (int)((size_t)nsplit * T * E * sizeof(float)), 0x00020000);
    const int E4 = E >> 2;
    for (int q0 = tid; q0 < 16 * E4; q0 += 1024) {
      f32x4 u[2][8];
      int qr[2], qe[2];
      bool ok[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int q = q0 + 512 * p;
        qr[p] = q / E4;
        qe[p] = q - qr[p] * E4;
        ok[p] = q < 16 * E4 && t0 + qr[p] < T;
#pragma unroll
        for (int sp = 0; sp < 8; ++sp) {
          u[p][sp] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (ok[p] && sp < nsplit) {
            const int off = (int)((((size_t)sp * T + t0 + qr[p]) * E + 4 * qe[p]) * sizeof(float));
            u[p][sp] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 16));   // 16: sc1
          }
        }
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (!ok[p]) continue;
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sp = 0; sp < 8; ++sp)
          if (sp < nsplit) v += u[p][sp];
#pragma unroll
        for (int c = 0; c < 4; ++c) lg_s[qr[p]][4 * qe[p] + c] = v[c];
      }
    }
  } else {
  for (int idx = tid; idx < 16 * E; idx += 512) {
    const int r = idx / E, e = idx % E;
    const int t = t0 + r;
    if (t >= T) continue;
    float* p = part + (size_t)t * E + e;
    const size_t stride = (size_t)T * E;
    float v = 0.f;
    int sp = 0;
    for (; sp + 8 <= nsplit; sp += 8) {
      float q[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)   // device-scope loads: not served from a stale cache line
        q[u] = __hip_atomic_load(p + (size_t)(sp + u) * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
      for (int u = 0; u < 8; ++u) v += q[u];
    }
    for (; sp < nsplit; ++sp)
      v += __hip_atomic_load(p + (size_t)sp * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lg_s[r][e] = v;
  }
  }
  __syncthreads();
  for (int r = wave; r < 16; r += kLastWaves) {
    const int t = t0 + r;
    if (t >= T) break;
    float lg[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = lane + 64 * c;
      lg[c] = e < E ? lg_s[r][e] : 0.f;
    }
    route_token(lg, t, o);
  }
  if (tid == 0) __hip_atomic_store(&ctr[blockIdx.x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // next call
}

// ---- many tokens: LDS-staged gate GEMM
//
// For hundreds of tokens and more the gate GEMM is a plain [T, H] x [H, E]
// product, and what matters is reading x once at full bandwidth and the
// gate weights as few times as possible.  A workgroup (4 waves) owns TT
// tokens and all EP >= E experts (so the weights are read T / TT times, not
// T / 16) over a K range; K advances in 128-byte slices (64 values) that go
// global -> LDS with direct 16-byte loads into a ring of NST stages, NST - 1
// slices ahead of the MFMAs, one barrier per slice.  LDS rows are 128 bytes
// with 16-byte chunk c of row r at chunk c ^ (r & 7) (conflict-free fragment
// reads).  The waves split the tile WT x WE ways (tokens x experts).  With
// several K ranges (too few token tiles to fill the device) each writes fp32
// partial logits that the reduce kernel sums in range order; with one, the
// workgroup selects in place.

template <int N>
__device__ __forceinline__ void gate_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// vmcnt <= ahead * LP for a wave-uniform ahead in [0, 14]
template <int LP>
__device__ __forceinline__ void gate_wait_ahead(int ahead) {
#define MOE_GW(A)                                  \
  case A:                                          \
    gate_wait_vmcnt<(A * LP < 64 ? A * LP : 0)>(); \
    break;
  switch (ahead) {
    MOE_GW(1) MOE_GW(2) MOE_GW(3) MOE_GW(4) MOE_GW(5) MOE_GW(6) MOE_GW(7)
    MOE_GW(8) MOE_GW(9) MOE_GW(10) MOE_GW(11) MOE_GW(12) MOE_GW(13) MOE_GW(14)
    default: gate_wait_vmcnt<0>(); break;
  }
#undef MOE_GW
}

template <int EP, int TT, int WE, int NST>
struct GateCfg {
  static constexpr int SL = 128;                  // bytes of K per slice and row
  static constexpr int ROWS = TT + EP;            // LDS rows per stage: tokens, then experts
  static constexpr int STAGE = ROWS * SL;
  static constexpr int LP = ROWS * SL / 4096;     // 16-byte loads per thread per slice
  static constexpr int WT = 4 / WE;               // waves along tokens
  static constexpr int MT = TT / WT / 16;         // 16-token tiles per wave
  static constexpr int NT = EP / WE / 16;         // 16-expert tiles per wave
  static constexpr int LDW = EP + 4;              // row stride of the fused path's logit tile
  static constexpr size_t LDS_BYTES =
      (size_t)NST * STAGE > (size_t)TT * LDW * 4 ? (size_t)NST * STAGE : (size_t)TT * LDW * 4;
  static_assert(ROWS % 32 == 0 && WE * WT == 4 && MT * WT * 16 == TT && NT * WE * 16 == EP, "tile shape");
  static_assert((NST - 2) * LP < 64 && NST - 2 <= 14, "wait counts");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  __device__ static __forceinline__ int off(int r, int c) { return r * SL + ((c ^ (r & 7)) << 4); }
};

// Direct loads of slice kt (relative to the range start) into stage st.
template <typename C>
__device__ __forceinline__ void gate_issue(uint8_t* smem, const uint8_t* const* src, int kt, int st, int wave) {
  uint8_t* dst = smem + st * C::STAGE + wave * 1024;
  const size_t koff = (size_t)kt * C::SL;
#pragma unroll
  for (int i = 0; i < C::LP; ++i) {
    const uint8_t* g = src[i] + koff;
    uint8_t* l = dst + i * 4096;
    __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
  }
}

template <int EP, int TT, int WE, int NST, bool FUSED>
__global__ __launch_bounds__(256, 1) void gate_tile_kernel(const uint8_t* __restrict__ x,
                                                           const uint8_t* __restrict__ wg, int T, int H, int nsplit,
                                                           float* __restrict__ part, RouteOut o) {
  using C = GateCfg<EP, TT, WE, NST>;
  using F = Frag<MOE_BF16>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int wt = wave / WE, we = wave % WE;
  const int t0 = blockIdx.x * TT;
  const int s = blockIdx.y;
  const int nsl = H * 2 / C::SL;
  const int k0 = (int)((long long)nsl * s / nsplit), k1 = (int)((long long)nsl * (s + 1) / nsplit);
  const int nk = k1 - k0;
  const int E = o.E;
  const size_t rowbytes = (size_t)H * 2;

  // Load i of thread tid fills LDS row (256 i + tid) / 8 at physical chunk
  // tid % 8, which holds logical chunk (tid % 8) ^ (row % 8).  Token rows
  // past T and expert rows past E repeat the last valid row (never stored).
  const uint8_t* src[C::LP];
#pragma unroll
  for (int i = 0; i < C::LP; ++i) {
    const int r = (i * 256 + tid) >> 3;
    const int lc = (tid & 7) ^ (r & 7);
    const uint8_t* base = r < TT ? x + (size_t)min(t0 + r, T - 1) * rowbytes
                                 : wg + (size_t)min(r - TT, E - 1) * rowbytes;
    src[i] = base + (size_t)k0 * C::SL + lc * 16;
  }

  f32x4 acc[C::MT][C::NT];
#pragma unroll
  for (int i = 0; i < C::MT; ++i)
#pragma unroll
    for (int j = 0; j < C::NT; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < nk) gate_issue<C>(smem, src, p, p, wave);
  for (int kt = 0; kt < nk; ++kt) {
    gate_wait_ahead<C::LP>(min(nk - 1 - kt, NST - 2));   // this thread's loads of slice kt have landed
    asm volatile("s_barrier" ::: "memory");              // everyone's have; stage (kt - 1) % NST is free
    if (kt + NST - 1 < nk) gate_issue<C>(smem, src, kt + NST - 1, (kt + NST - 1) % NST, wave);
    const uint8_t* la = smem + (kt % NST) * C::STAGE;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x4 fa[C::MT], fb[C::NT];
#pragma unroll
      for (int i = 0; i < C::MT; ++i)
        fa[i] = *reinterpret_cast<const i32x4*>(&la[C::off((wt * C::MT + i) * 16 + row, ks * 4 + grp)]);
#pragma unroll
      for (int j = 0; j < C::NT; ++j)
        fb[j] = *reinterpret_cast<const i32x4*>(&la[C::off(TT + (we * C::NT + j) * 16 + row, ks * 4 + grp)]);
#pragma unroll
      for (int i = 0; i < C::MT; ++i)
#pragma unroll
        for (int j = 0; j < C::NT; ++j) F::mma(acc[i][j], fa[i], fb[j]);
    }
  }

  // acc[i][j][q]: token t0 + (wt MT + i) 16 + 4 grp + q, expert (we NT + j) 16 + row
  if constexpr (!FUSED) {
#pragma unroll
    for (int i = 0; i < C::MT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + (wt * C::MT + i) * 16 + 4 * grp + q;
        if (t >= T) continue;
        float* pr = part + ((size_t)s * T + t) * E;
#pragma unroll
        for (int j = 0; j < C::NT; ++j) {
          const int e = (we * C::NT + j) * 16 + row;
          if (e < E) pr[e] = acc[i][j][q];
        }
      }
  } else {
    float* lg_s = reinterpret_cast<float*>(smem);   // [TT][LDW]
    __syncthreads();                                 // every wave is done with the stages
#pragma unroll
    for (int i = 0; i < C::MT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < C::NT; ++j)
          lg_s[((wt * C::MT + i) * 16 + 4 * grp + q) * C::LDW + (we * C::NT + j) * 16 + row] = acc[i][j][q];
    __syncthreads();
    for (int r = wave; r < TT; r += 4) {
      const int t = t0 + r;
      if (t >= T) break;
      float lg[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = lane + 64 * c;
        lg[c] = e < E ? lg_s[r * C::LDW + e] : 0.f;
      }
      route_token(lg, t, o);
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

namespace {

// Shape of the LDS-staged gate GEMM for this layer, or ep = 0 for the
// 16-token kernel (few tokens, or fp32 activations).
struct GateShape {
  int ep, tt, nst;
};
constexpr int kGateTileMinT = 512;

GateShape gate_shape(const moe_cfg& c) {
  if (c.act_dtype != MOE_BF16 || c.T < kGateTileMinT || c.H % 64 != 0) return {0, 0, 0};
  if (c.E <= 32) return {32, 128, 6};
  if (c.E <= 64) return {64, 128, 5};
  if (c.E <= 128) return {128, 128, 4};
  return {256, 64, 3};
}

}  // namespace

// The one-launch router for up to kLastMaxTiles token tiles (see
// gate_last_kernel): K splits so that each wave keeps at least two
// fragments, at most 8 (the last workgroup reads 8 partials per logit).
// Measured at H = 7168, E = 256 (router us, split + reduce launches before):
// 16 tokens 8 splits 21.3-22.3 (25.5 before), 4 splits 24.3-24.6;
// 256 tokens 8 splits 26.8, 4 splits 24.9-25.5 (28.3-30.0 before).
static int last_splits(const moe_cfg& c) {
  const int kf = c.act_dtype == MOE_F32 ? Frag<MOE_F32>::KF : Frag<MOE_BF16>::KF;
  const int cap = ceil_div(c.T, kTokTile) <= 4 ? 8 : 4;   // at most 8: the last workgroup's loads
  const int s = c.H / kf / (2 * kLastWaves);
  return s < 1 ? 1 : (s > cap ? cap : s);
}

static bool use_last(const moe_cfg& c) {
  return gate_shape(c).ep == 0 && ceil_div(c.T, kTokTile) <= kLastMaxTiles;
}

int route_splits(const moe_cfg& c) {
  if (use_last(c)) return last_splits(c);
  const GateShape gs = gate_shape(c);
  if (gs.ep > 0) {   // fill the device with (token tile, K range) workgroups, >= 2 NST slices per range
    const int tiles = ceil_div(c.T, gs.tt);
    if (tiles >= 256) return 1;
    const int cap = c.H / 64 / (2 * gs.nst);
    const int s = ceil_div(256, tiles);
    return s < cap ? s : (cap > 1 ? cap : 1);
  }
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
  if (use_last(c)) return (size_t)s * c.T * c.E * sizeof(float);   // partials of every expert group
  return s > 1 ? (size_t)s * c.T * c.E * sizeof(float) : 0;
}

static hipError_t launch_reduce(const moe_cfg& c, const float* part, int s, const RouteOut& o, hipStream_t st) {
  MOE_LAUNCH("route_reduce_select", route_reduce_kernel, dim3(c.T), dim3(256), 0, st, part, c.T, s, o);
  return hipGetLastError();
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

template <int EP, int TT, int WE, int NST, bool FUSED>
static hipError_t launch_gate_tile(const moe_cfg& c, dim3 grid, const uint8_t* xb, const uint8_t* wb, int s,
                                   float* part, const RouteOut& o, hipStream_t st) {
  using C = GateCfg<EP, TT, WE, NST>;
  hipError_t e = moe::ensure_dynamic_lds(reinterpret_cast<const void*>(&gate_tile_kernel<EP, TT, WE, NST, FUSED>),
                                          (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  MOE_LAUNCH("route_gate_tiled", (gate_tile_kernel<EP, TT, WE, NST, FUSED>), grid, dim3(256), C::LDS_BYTES, st, xb,
             wb, c.T, c.H, s, part, o);
  return hipGetLastError();
}

template <bool FUSED>
static hipError_t launch_gate_tile_shape(const moe_cfg& c, const GateShape& gs, dim3 grid, const uint8_t* xb,
                                         const uint8_t* wb, int s, float* part, const RouteOut& o, hipStream_t st) {
  switch (gs.ep) {
    case 32: return launch_gate_tile<32, 128, 1, 6, FUSED>(c, grid, xb, wb, s, part, o, st);
    case 64: return launch_gate_tile<64, 128, 1, 5, FUSED>(c, grid, xb, wb, s, part, o, st);
    case 128: return launch_gate_tile<128, 128, 2, 4, FUSED>(c, grid, xb, wb, s, part, o, st);
    default: return launch_gate_tile<256, 64, 4, 3, FUSED>(c, grid, xb, wb, s, part, o, st);
  }
}

hipError_t launch_route(const moe_cfg& c, const void* x, const void* wg, const float* bias, int32_t* idx,
                        float* w, float* part, int32_t* ctr, hipStream_t st) {
  RouteOut o{bias, idx, w, c.E, c.k, c.score, c.routed_scale, c.n_group, c.topk_group};
  if (use_last(c)) {
    const int s = last_splits(c);
    const dim3 grid(ceil_div(c.T, kTokTile), ceil_div(c.E, kLastEG) * s);
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    const uint8_t* wb = static_cast<const uint8_t*>(wg);
    if (c.act_dtype == MOE_F32)
      MOE_LAUNCH("route_gate_last", gate_last_kernel<MOE_F32>, grid, dim3(512), 0, st, xb, wb, c.T, c.H, s, part, ctr, o);
    else
      MOE_LAUNCH("route_gate_last", gate_last_kernel<MOE_BF16>, grid, dim3(512), 0, st, xb, wb, c.T, c.H, s, part, ctr, o);
    return hipGetLastError();
  }
  const GateShape gs = gate_shape(c);
  if (gs.ep > 0) {
    const int s = route_splits(c);
    const dim3 grid(ceil_div(c.T, gs.tt), s);
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    const uint8_t* wb = static_cast<const uint8_t*>(wg);
    hipError_t e = s == 1 ? launch_gate_tile_shape<true>(c, gs, grid, xb, wb, 1, nullptr, o, st)
                          : launch_gate_tile_shape<false>(c, gs, grid, xb, wb, s, part, o, st);
    if (e != hipSuccess || s == 1) return e;
    return launch_reduce(c, part, s, o, st);
  }
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
  return launch_reduce(c, part, s, o, st);
}

}  // namespace moe
