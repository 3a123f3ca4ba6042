// Expert FFNs as grouped GEMMs (steps: SwiGLU up/gate GEMM, down GEMM,
// shared expert).
//
// Perplexity's "Lower latency and higher throughput with multi-node DeepSeek
// deployment" states the grouped GEMM (section "GroupGEMM": group i computes
// [m_i, k] x [k, n]) and argues from its roofline that it is bandwidth-bound
// while per-expert row counts are small and compute-bound in prefill (sections
// "GroupGEMM" and "Future work"), and that under graph capture the kernels
// must read the per-expert token counts from the routing on the device
// (section "Quantization", MoE-router paragraph).  So:
//
//   plan kernel   reads offsets[] on the device and sorts the groups (the E
//                 routed experts plus the shared expert as group E) into two
//                 regimes: "skinny" groups with 1..kSkinnyRows rows and "fat"
//                 groups, cut into kBM-row tiles.
//   skinny GEMM   one wave streams 16-row tiles of an expert's weight matrix
//                 straight from HBM into MFMA B registers (each weight byte is
//                 read once) against the group's <= 32 rows, which stay hot in
//                 L2.  Bandwidth-bound decode regime.
//   fat GEMM      128 x 128 output tiles per workgroup, K staged through LDS
//                 in double-buffered 128-byte slices (XOR-swizzled 16-byte
//                 chunks), 2 x 2 waves each computing 64 x 64 with 16x16 MFMAs.
//                 Compute-bound prefill regime.
//
// GEMM1 (mode 1) produces h = SiLU(A W1^T) * (A W3^T): every output tile holds
// matching gate and up columns (16-column blocks interleaved gate, up, gate,
// up), so SwiGLU is applied in registers.  GEMM2 (mode 2) is the down
// projection into y_sorted (routed) or y_shared.
//
// FP8 E4M3 weights carry one fp32 scale per row per 128 K-values and the
// activations one scale per row per 128: each 128-wide K block is one
// 16x16x128 MFMA with unit block exponents, promoted to fp32 with
// scale_a[row] * scale_w[col] and accumulated on the vector ALU.

#include "moe_common.h"
#include "moe_launch.h"

namespace {

constexpr int kSkinnyRows = 32;  // groups with <= this many rows take the skinny path
constexpr int kTileRows = 256;   // rows per tile of the tiled grouped GEMM
constexpr int kPlanHead = 4;     // plan: [0..2] skinny list sizes (<=8, <=16, <=32 rows), [3] fat tiles

struct Args {
  int T, H, E, k, I, P;
  int has_shared;
  int qb;                       // fp8 block (128)
  const uint8_t* a1;            // GEMM1 A rows: x or fp8 codes of x, [T, H]
  const float* a1s;             // fp8: x scales [T, H/qb]
  const int32_t* offsets;
  const int32_t* sorted_pair;
  const uint8_t* w13;
  const float* w13s;
  const uint8_t* ws13;
  const float* ws13s;
  const uint8_t* w2;
  const float* w2s;
  const uint8_t* ws2;
  const float* ws2s;
  uint8_t* h;                   // GEMM1 out [P+T, I]
  const uint8_t* a2;            // GEMM2 A rows: h or fp8 codes of h, [P+T, I]
  const float* a2s;             // fp8: h scales [P+T, I/qb]
  uint8_t* y_sorted;            // act dtype (fp32 when DT is fp32, else bf16)
  uint8_t* y_shared;
  const int32_t* plan;          // see ffn_plan_kernel: list sizes, 3 skinny lists of G, fat (group,row0) pairs
  int G;
  int shared_only;              // tiled launch over the shared expert's row tiles instead of the plan's fat list
};

struct Group {
  int m;         // rows
  int slot0;     // first row in the [P+T] row space of h (routed: offsets[g]; shared: P)
  bool routed;
};

__device__ __forceinline__ Group group_of(const Args& a, int g) {
  Group r;
  if (g < a.E) {
    r.slot0 = a.offsets[g];
    r.m = a.offsets[g + 1] - r.slot0;
    r.routed = true;
  } else {
    r.slot0 = a.P;
    r.m = a.T;
    r.routed = false;
  }
  return r;
}

// Token (row of x) feeding row r of group g in GEMM1.
__device__ __forceinline__ int gemm1_src_row(const Args& a, const Group& gr, int r) {
  return gr.routed ? a.sorted_pair[gr.slot0 + r] / a.k : r;
}

template <int DT> struct HOut;  // element type of h
template <> struct HOut<MOE_F32> { static constexpr int ESZ = 4; };
template <> struct HOut<MOE_BF16> { static constexpr int ESZ = 2; };
template <> struct HOut<MOE_FP8_E4M3> { static constexpr int ESZ = 4; };  // fp32, quantised afterwards

template <int DT>
__device__ __forceinline__ void store_h(uint8_t* h, size_t idx, float v) {
  if constexpr (DT == MOE_BF16)
    reinterpret_cast<uint16_t*>(h)[idx] = f32_to_bf16(v);
  else
    reinterpret_cast<float*>(h)[idx] = v;
}

// Expert outputs are stored in the activation dtype: fp32 for the fp32 layer,
// bf16 for bf16 and fp8 weights.
template <int DT>
__device__ __forceinline__ void store_y(uint8_t* y, size_t idx, float v) {
  if constexpr (DT == MOE_F32)
    reinterpret_cast<float*>(y)[idx] = v;
  else
    reinterpret_cast<uint16_t*>(y)[idx] = f32_to_bf16(v);
}

// ------------------------------------------------------------------ plan

__global__ __launch_bounds__(512) void ffn_plan_kernel(Args a) {
  __shared__ int sk[3][512];
  __shared__ int ft[512];
  const int g = threadIdx.x;
  int m = 0;
  if (g < a.G) m = g < a.E ? a.offsets[g + 1] - a.offsets[g] : a.T;
  // skinny class: 0 for 1..8 rows, 1 for 9..16, 2 for 17..32 (a skinny shared
  // expert has a launch of its own and is in no list)
  const bool shared = g == a.E;
  const int cls = (m > 0 && m <= kSkinnyRows && !shared) ? (m <= 8 ? 0 : m <= 16 ? 1 : 2) : -1;
  // the shared expert is never in the lists: it has launches of its own
  const int tiles = m > kSkinnyRows && !shared ? (m + kTileRows - 1) / kTileRows : 0;
#pragma unroll
  for (int c = 0; c < 3; ++c) sk[c][g] = cls == c ? 1 : 0;
  ft[g] = tiles;
  __syncthreads();
  for (int d = 1; d < 512; d <<= 1) {
    int v[3];
#pragma unroll
    for (int c = 0; c < 3; ++c) v[c] = g >= d ? sk[c][g - d] : 0;
    const int v2 = g >= d ? ft[g - d] : 0;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < 3; ++c) sk[c][g] += v[c];
    ft[g] += v2;
    __syncthreads();
  }
  int32_t* plan = const_cast<int32_t*>(a.plan);
  if (g == 511) {
#pragma unroll
    for (int c = 0; c < 3; ++c) plan[c] = sk[c][511];
    plan[3] = ft[511];
  }
  if (cls >= 0) plan[kPlanHead + cls * a.G + sk[cls][g] - 1] = g;
  const int t0 = ft[g] - tiles;
  int32_t* fat = plan + kPlanHead + 3 * a.G;
  for (int i = 0; i < tiles; ++i) {
    fat[2 * (t0 + i)] = g;
    fat[2 * (t0 + i) + 1] = i * kTileRows;
  }
}

// ------------------------------------------------------------------ skinny grouped GEMM
//
// Streaming layout.  A weight row is read in 128-byte windows (one cache
// line).  One wave load instruction covers 8 weight rows x one window: lane l
// reads row (l % 8), 16-byte chunk c(l) = 4 * ((l >> 3) & 1) + (l >> 4).  Fed
// as the B operand of a 16x16 MFMA, column n (lane l % 16) thus holds weight
// row n % 8, and columns n and n + 8 hold the two complementary 64-byte halves
// of the window.  The A operand mirrors this: M row m holds token m % 8 with
// the same chunk rule.  The diagonal 8x8 blocks of the 16x16 result are then
// the two K halves of the same (token, row) dot products and the off-diagonal
// blocks are discarded: out[t][r] = C[t][r] + C[t+8][r+8], which sits in lanes
// L and L ^ 40.  Half of each MFMA is wasted, which costs nothing in this
// bandwidth-bound regime, and every load instruction reads whole cache lines.

constexpr int kSkNT = 8;  // 8-row weight tiles per routed skinny item (even: gate/up halves in GEMM1)

// Weights are read exactly once: nontemporal loads keep them from displacing
// the reused activation rows in the caches.
__device__ __forceinline__ i32x4 ldw16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}

__device__ __forceinline__ int sk_chunk(int lane) { return 4 * ((lane >> 3) & 1) + (lane >> 4); }

// One pass over the full K for NTP of the wave's NT weight tiles (pass p),
// against MT M tiles of 8 tokens (MT * 8 >= group rows).  Rows beyond the
// group's count are clamped to its last row: their results are never stored,
// so the K loop carries no per-lane predicates or branches.  U windows per
// loop trip give NTP * U = 8 independent weight loads per lane.
//
// Split K (KS > 1): the KS waves of a workgroup share the item, wave `ks`
// takes windows [ks*nwin/KS, (ks+1)*nwin/KS); partial accumulators meet in
// LDS and wave 0 adds them in slice order (fixed order: reproducible) before
// the epilogue.
template <int DT, int MODE, int MT, int NT, int NTP, int U, int KS>
__device__ __forceinline__ void skinny_pass(const Args& a, const Group& gr, int g, int it, int p, int lane,
                                            int ks, f32x4* red) {
  using F = Frag<DT>;
  constexpr bool FP8 = DT == MOE_FP8_E4M3;
  const int r8 = lane & 7;
  const int ch16 = sk_chunk(lane) * 16;
  const int cols_per_item = MODE == 1 ? 4 * NT : 8 * NT;   // h columns (GEMM1) or y columns (GEMM2)
  const int K = MODE == 1 ? a.H : a.I;
  const size_t krow = (size_t)K * F::ESZ;
  const int nwin = (int)(krow / 128);
  const int w_begin = KS > 1 ? (int)((long long)nwin * ks / KS) : 0;
  const int w_end = KS > 1 ? (int)((long long)nwin * (ks + 1) / KS) : nwin;

  const uint8_t* abase = MODE == 1 ? a.a1 : a.a2;
  int arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = min(mt * 8 + r8, gr.m - 1);
    arow[mt] = MODE == 1 ? gemm1_src_row(a, gr, r) : gr.slot0 + r;
  }
  const uint8_t* wbase;
  const float* wsbase = nullptr;
  if (MODE == 1) {
    wbase = gr.routed ? a.w13 + (size_t)g * 2 * a.I * krow : a.ws13;
    if (FP8) wsbase = gr.routed ? a.w13s + (size_t)g * 2 * a.I * nwin : a.ws13s;
  } else {
    wbase = gr.routed ? a.w2 + (size_t)g * a.H * krow : a.ws2;
    if (FP8) wsbase = gr.routed ? a.w2s + (size_t)g * a.H * nwin : a.ws2s;
  }
  // tile j of this pass -> tile index in the item (GEMM1: first half gate, second half up)
  int wrow[NTP];
#pragma unroll
  for (int j = 0; j < NTP; ++j) {
    if (MODE == 1) {
      const int jg = j < NTP / 2 ? p * (NTP / 2) + j : p * (NTP / 2) + j - NTP / 2;   // gate-tile index
      wrow[j] = (j < NTP / 2 ? 0 : a.I) + it * cols_per_item + 8 * jg + r8;
    } else {
      wrow[j] = it * cols_per_item + 8 * (p * NTP + j) + r8;
    }
  }
  const uint8_t* pb[NTP];
#pragma unroll
  for (int j = 0; j < NTP; ++j) pb[j] = wbase + (size_t)wrow[j] * krow + ch16;
  const uint8_t* pa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) pa[mt] = abase + (size_t)arow[mt] * krow + ch16;

  f32x4 acc[MT][NTP];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NTP; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (!FP8) {
    int w = w_begin;
    for (; w + U <= w_end; w += U) {
      i32x4 b[U][NTP], av[U][MT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t off = (size_t)(w + u) * 128;
#pragma unroll
        for (int j = 0; j < NTP; ++j) b[u][j] = ldw16(pb[j] + off);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) av[u][mt] = ld16(pa[mt] + off);
      }
      // Keep every load of the trip ahead of its MFMAs: left alone, the
      // scheduler interleaves them to shorten live ranges and waits on each
      // load in turn, which leaves few bytes in flight per wave.
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < NTP; ++j) F::mma(acc[mt][j], av[u][mt], b[u][j]);
    }
    for (; w < w_end; ++w) {
      const size_t off = (size_t)w * 128;
      i32x4 b[NTP];
#pragma unroll
      for (int j = 0; j < NTP; ++j) b[j] = ldw16(pb[j] + off);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const i32x4 av = ld16(pa[mt] + off);
#pragma unroll
        for (int j = 0; j < NTP; ++j) F::mma(acc[mt][j], av, b[j]);
      }
    }
  } else {
    // One 128-byte window is one fp8 scale block.  Scales of the C rows this
    // lane holds (token (4*(lane>>4)+i) % 8 of each M tile) and of its column's row.
    const float* sbase = MODE == 1 ? a.a1s : a.a2s;
    int sa_row[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = min(mt * 8 + ((4 * (lane >> 4) + i) & 7), gr.m - 1);
        sa_row[mt][i] = (MODE == 1 ? gemm1_src_row(a, gr, r) : gr.slot0 + r) * nwin;
      }
    // U windows per trip: all loads of the trip are issued before its MFMAs.
    constexpr int UF = MT >= 4 ? (U < 2 ? U : 2) : U;
    int w = w_begin;
    for (; w < w_end; w += UF) {
      i32x4 b[UF][NTP], av[UF][MT];
      float sw[UF][NTP], sa[UF][MT][4];
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        const int wu = min(w + u, w_end - 1);   // a short last trip recomputes its last window, not added
        const size_t off = (size_t)wu * 128;
#pragma unroll
        for (int j = 0; j < NTP; ++j) b[u][j] = ldw16(pb[j] + off);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) av[u][mt] = ld16(pa[mt] + off);
#pragma unroll
        for (int j = 0; j < NTP; ++j) sw[u][j] = wsbase[(size_t)wrow[j] * nwin + wu];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sa[u][mt][i] = sbase[(size_t)sa_row[mt][i] + wu];
      }
      __builtin_amdgcn_sched_barrier(0);   // all loads of the trip before its MFMAs
#pragma unroll
      for (int u = 0; u < UF; ++u) {
        if (u > 0 && w + u >= w_end) break;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < NTP; ++j) {
            f32x4 pr = {0.f, 0.f, 0.f, 0.f};
            // a 16-byte chunk is 16 fp8 values: two 16x16x32 MFMAs (8 bytes per lane each)
            pr = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(((const long*)&av[u][mt])[0], ((const long*)&b[u][j])[0], pr, 0, 0, 0);
            pr = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(((const long*)&av[u][mt])[1], ((const long*)&b[u][j])[1], pr, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][j][i] = fmaf(pr[i], sa[u][mt][i] * sw[u][j], acc[mt][j][i]);
          }
      }
    }
  }

  if constexpr (KS > 1) {
    // red: [KS-1][MT*NTP][64] partial accumulators of waves 1..KS-1
    if (ks > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NTP; ++j) red[((ks - 1) * MT * NTP + mt * NTP + j) * 64 + lane] = acc[mt][j];
    }
    __syncthreads();
    if (ks == 0) {
      for (int q = 0; q < KS - 1; ++q)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int j = 0; j < NTP; ++j) acc[mt][j] += red[(q * MT * NTP + mt * NTP + j) * 64 + lane];
    }
    __syncthreads();
    if (ks > 0) return;
  }

  // Fold the two K halves: lanes L = 16*h + r (h < 2, r < 8) end up holding
  // tokens 4*h + i (i = 0..3) of each M tile for weight row r of each tile.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < NTP; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[mt][j][i] += __shfl_xor(acc[mt][j][i], 40, 64);
  if ((lane & 8) || lane >= 32) return;
  const int hh = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mt * 8 + 4 * hh + i;
      if (r >= gr.m) continue;
      if (MODE == 1) {
        const size_t hrow = (size_t)(gr.slot0 + r) * a.I;
#pragma unroll
        for (int j = 0; j < NTP / 2; ++j) {
          const float gv = acc[mt][j][i], uv = acc[mt][j + NTP / 2][i];
          store_h<DT>(a.h, hrow + it * cols_per_item + 8 * (p * (NTP / 2) + j) + r8, silu(gv) * uv);
        }
      } else {
        uint8_t* ybase = gr.routed ? a.y_sorted : a.y_shared;
        const size_t yrow = (size_t)(gr.routed ? gr.slot0 + r : r) * a.H;
#pragma unroll
        for (int j = 0; j < NTP; ++j) store_y<DT>(ybase, yrow + it * cols_per_item + 8 * (p * NTP + j) + r8, acc[mt][j][i]);
      }
    }
  }
}

// All NT tiles of an item with MT M tiles: NT / NTP passes.
template <int DT, int MODE, int MT, int NT, int KS>
__device__ __forceinline__ void skinny_tile(const Args& a, const Group& gr, int g, int it, int lane, int ks,
                                            f32x4* red) {
  constexpr int NTP = MT == 1 ? NT : (NT / MT >= 2 ? NT / MT : 2);
  constexpr int U0 = 8 / NTP > 0 ? 8 / NTP : 1;
  constexpr int U = MT >= 4 && U0 > 2 ? 2 : U0;
  for (int p = 0; p < NT / NTP; ++p) skinny_pass<DT, MODE, MT, NT, NTP, U, KS>(a, gr, g, it, p, lane, ks, red);
}

// Routed skinny groups of class CLS (MT = 1, 2, 4 M tiles of 8 tokens).
// One wave = one work item (group, column block of kSkNT weight tiles) in a
// single pass over K; waves past the class's list exit at once.  Every class
// uses the same wide items: each activation fragment then serves 8 weight
// tiles, which keeps the activation re-reads (one per item) a small share of
// the load instructions even at 32 rows.
template <int DT, int MODE, int CLS>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(Args a) {
  constexpr int MT = 1 << CLS;
  constexpr int NT = kSkNT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cols_per_item = MODE == 1 ? 4 * NT : 8 * NT;
  const int items = (MODE == 1 ? a.I : a.H) / cols_per_item;
  // XCD-aware order: workgroups go to the 8 XCDs round-robin (blockIdx % 8),
  // so XCD x takes the contiguous range x * per_xcd ... of the class's real
  // work.  The items of a group then run on one or two XCDs and its
  // activation rows, re-read by every item, stay in that XCD's L2 instead of
  // being fetched into all eight.  The grid is a multiple of 8 and at least
  // 8 * per_xcd workgroups.
  const int real_wg = (a.plan[CLS] * items + 3) >> 2;
  const int per_xcd = (real_wg + 7) >> 3;
  const int local = blockIdx.x >> 3;
  if (local >= per_xcd) return;
  const int item = ((blockIdx.x & 7) * per_xcd + local) * 4 + wave;
  const int gi = item / items;
  if (gi >= a.plan[CLS]) return;
  const int g = a.plan[kPlanHead + CLS * a.G + gi];
  const int it = item - gi * items;
  const Group gr = group_of(a, g);
  skinny_pass<DT, MODE, MT, NT, NT, 1, 1>(a, gr, g, it, 0, lane, 0, nullptr);
}

// The shared expert when T <= kSkinnyRows: its row count is known on the
// host, so its launch is sized exactly, with narrow items (kShNT tiles) and
// the K range split over the kShKS waves of each workgroup.
constexpr int kShNT = 2;
constexpr int kShKS = 8;

template <int DT, int MODE, int MT>
__global__ __launch_bounds__(64 * kShKS) void ffn_shared_skinny_kernel(Args a) {
  constexpr int NTP = MT == 1 ? kShNT : (kShNT / MT >= 2 ? kShNT / MT : 2);
  __shared__ f32x4 red[(kShKS - 1) * MT * NTP * 64];
  const int lane = threadIdx.x & 63, ks = threadIdx.x >> 6;
  const Group gr = group_of(a, a.E);
  skinny_tile<DT, MODE, MT, kShNT, kShKS>(a, gr, a.E, blockIdx.x, lane, ks, red);
}

// ------------------------------------------------------------------ tiled grouped GEMM
//
// 256 x 256 output tile per workgroup of 8 waves (4 along M x 2 along N, each
// 64 x 128 with 16x16 MFMAs).  K advances in slices of SL bytes per row: each
// slice of the 256 A rows and the 256 B rows goes global -> LDS directly (16
// bytes per lane per instruction) into an NST-deep ring of LDS stages, so the
// loads run NST - 1 slices ahead of the MFMAs and there is one barrier per
// slice.  bf16/fp32 use 64-byte slices with 4 stages; fp8 uses 128-byte
// slices (one scale block) with 2 stages.  LDS rows are SL bytes with 16-byte
// chunk c of row r stored at chunk c ^ swizzle(r), which keeps the fragment
// reads of 16 consecutive rows free of bank conflicts; the direct loads write
// chunks in lane order, so each lane fetches the global chunk that belongs
// at its position.  Waves whose 64 rows lie beyond the tile's valid rows skip
// their MFMAs.

constexpr int kTM = 256;                  // tile rows (tokens)
constexpr int kTN = 256;                  // tile columns (weight rows; GEMM1: 128 gate + 128 up)

template <int DT> struct TileCfg {
  static constexpr int SL = 128;                              // bytes of K per slice and row
  static constexpr int NST = 2;                               // LDS stages
  static constexpr int CPR = SL / 16;                         // 16-byte chunks per row
  static constexpr int STAGE = (kTM + kTN) * SL;              // bytes per stage (A then B)
  static constexpr int LPS = SL / 32;                         // direct loads per thread per slice, A and B each
  static constexpr int ROWS_PER_INSTR = 1024 / SL;            // rows one wave instruction fills
  __device__ static __forceinline__ int off(int r, int c) {
    const int sw = SL == 128 ? (r & 7) : ((r >> 2) & 3);
    return r * SL + ((c ^ sw) << 4);
  }
};

// s_waitcnt that waits for vmcnt <= n only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Issue the direct global -> LDS loads of slice kt into stage st (and, for
// fp8, store the scale fetched one slice earlier and fetch the next one).
template <int DT>
__device__ __forceinline__ void tile_issue(uint8_t* smem, const uint8_t* const* ga, const uint8_t* const* gb, int kt,
                                           int st, int wave, int tid, int nkt, float* lds_s, const float* gs,
                                           float& rs) {
  using C = TileCfg<DT>;
  const size_t off = (size_t)kt * C::SL;
  uint8_t* la = smem + st * C::STAGE + wave * C::LPS * 1024;
  uint8_t* lb = smem + st * C::STAGE + kTM * C::SL + wave * C::LPS * 1024;
#pragma unroll
  for (int i = 0; i < C::LPS; ++i) {
    __builtin_amdgcn_global_load_lds(ga[i] + off, la + i * 1024, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(gb[i] + off, lb + i * 1024, 16, 0, 0);
  }
  if constexpr (DT == MOE_FP8_E4M3) {
    lds_s[st * (kTM + kTN) + tid] = rs;
    if (kt + 1 < nkt) rs = gs[kt + 1];            // consumed one slice later
  }
}

template <int DT, int MODE>
__global__ __launch_bounds__(512, 1) void ffn_fat_kernel(Args a, int ntn) {
  using F = Frag<DT>;
  using C = TileCfg<DT>;
  constexpr bool FP8 = DT == MOE_FP8_E4M3;
  constexpr int SL = C::SL, NST = C::NST, LPS = C::LPS, RPI = C::ROWS_PER_INSTR;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  float* lds_s = reinterpret_cast<float*>(smem + NST * C::STAGE);   // fp8: [NST][kTM + kTN]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int tile = blockIdx.x / ntn;
  const int nt = blockIdx.x - tile * ntn;
  int g, row0;
  if (a.shared_only) {              // the grid covers exactly ceil(T / kTM) row tiles of the shared expert
    g = a.E;
    row0 = tile * kTM;
  } else {
    if (tile >= a.plan[3]) return;
    const int32_t* fat = a.plan + kPlanHead + 3 * a.G;
    g = fat[2 * tile];
    row0 = fat[2 * tile + 1];
  }
  const Group gr = group_of(a, g);
  const int rows = min(kTM, gr.m - row0);
  const int K = MODE == 1 ? a.H : a.I;
  const size_t krow = (size_t)K * F::ESZ;
  const int nkt = (int)(krow / SL);
  const int nkb = FP8 ? K / a.qb : 0;

  const uint8_t* asrc = MODE == 1 ? a.a1 : a.a2;
  const uint8_t* wbase;
  const float* wsbase = nullptr;
  if (MODE == 1) {
    wbase = gr.routed ? a.w13 + (size_t)g * 2 * a.I * krow : a.ws13;
    if (FP8) wsbase = gr.routed ? a.w13s + (size_t)g * 2 * a.I * nkb : a.ws13s;
  } else {
    wbase = gr.routed ? a.w2 + (size_t)g * a.H * krow : a.ws2;
    if (FP8) wsbase = gr.routed ? a.w2s + (size_t)g * a.H * nkb : a.ws2s;
  }
  // Weight row held by LDS B row n; columns past N (a partial last column
  // tile) are clamped to the last valid row and never stored.
  auto b_wrow = [&](int n) -> int {
    if (MODE == 1) {
      const int blk = n >> 4;          // 16-row blocks alternate gate, up
      const int hc = min(nt * (kTN / 2) + (blk >> 1) * 16 + (n & 15), a.I - 1);
      return ((blk & 1) ? a.I : 0) + hc;
    }
    return min(nt * kTN + n, a.H - 1);
  };
  // This lane's direct-load sources.  Wave instruction i fills LDS rows
  // (wave * LPS + i) * RPI + lane / CPR, physical chunk lane % CPR.
  const uint8_t* ga[LPS];
  const uint8_t* gb[LPS];
#pragma unroll
  for (int i = 0; i < LPS; ++i) {
    const int r = (wave * LPS + i) * RPI + lane / C::CPR;
    const int pc = lane % C::CPR;
    const int lc = (C::off(r, pc) - r * SL) >> 4;   // the swizzle is an involution: logical chunk of physical pc
    const int rr = r < rows ? r : rows - 1;          // clamp: padded rows recompute a valid row, never stored
    const int src = MODE == 1 ? gemm1_src_row(a, gr, row0 + rr) : gr.slot0 + row0 + rr;
    ga[i] = asrc + (size_t)src * krow + lc * 16;
    gb[i] = wbase + (size_t)b_wrow(r) * krow + lc * 16;
  }
  // fp8 scales: thread tid < kTM loads A-row scale tid, the rest B-row scale tid - kTM
  const float* gs = nullptr;
  if constexpr (FP8) {
    if (tid < kTM) {
      const int r = tid < rows ? tid : rows - 1;
      const int src = MODE == 1 ? gemm1_src_row(a, gr, row0 + r) : gr.slot0 + row0 + r;
      gs = (MODE == 1 ? a.a1s : a.a2s) + (size_t)src * nkb;
    } else {
      gs = wsbase + (size_t)b_wrow(tid - kTM) * nkb;
    }
  }
  float rs = 0.f;                                  // fp8: scale for the next slice to issue
  if constexpr (FP8) rs = gs[0];

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int mval = min(4, max(0, (rows - wm * 64 + 15) >> 4));   // this wave's M tiles holding valid rows

#pragma unroll
  for (int p = 0; p < NST - 1; ++p)
    if (p < nkt) tile_issue<DT>(smem, ga, gb, p, p, wave, tid, nkt, lds_s, gs, rs);
  for (int kt = 0; kt < nkt; ++kt) {
    const int st = kt % NST;
    // wait until this thread's loads of slice kt have landed; later slices may stay in flight
    if constexpr (FP8) {
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      const int ahead = min(NST - 2, nkt - 1 - kt);   // slices issued after kt
      if (ahead >= 2) wait_vmcnt<4 * LPS>();
      else if (ahead == 1) wait_vmcnt<2 * LPS>();
      else wait_vmcnt<0>();
    }
    __syncthreads();                               // everyone's slice kt is in LDS; stage (kt-1) % NST is free
    if (kt + NST - 1 < nkt)
      tile_issue<DT>(smem, ga, gb, kt + NST - 1, (kt + NST - 1) % NST, wave, tid, nkt, lds_s, gs, rs);
    const uint8_t* la = smem + st * C::STAGE;
    const uint8_t* lb = la + kTM * SL;
    if constexpr (!FP8) {
      // Full tiles: all fragments of the slice are read first and the MFMAs
      // follow in the same straight-line block, so the compiler can start the
      // first half's MFMAs while the second half's reads are in flight.  Only
      // a group's last, partial tile takes the guarded path that skips M tiles.
      if (mval == 4) {
        i32x4 fa[SL / 64][4], fb[SL / 64][8];
#pragma unroll
        for (int fs = 0; fs < SL / 64; ++fs) {
#pragma unroll
          for (int j = 0; j < 8; ++j)
            fb[fs][j] = *reinterpret_cast<const i32x4*>(&lb[C::off(wn * 128 + j * 16 + row, fs * 4 + grp)]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            fa[fs][i] = *reinterpret_cast<const i32x4*>(&la[C::off(wm * 64 + i * 16 + row, fs * 4 + grp)]);
        }
#pragma unroll
        for (int fs = 0; fs < SL / 64; ++fs)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) F::mma(acc[i][j], fa[fs][i], fb[fs][j]);
        // Instruction order for the scheduler: the first half's 12 reads, then
        // the second half's 12 reads interleaved 1:2 with the first half's
        // MFMAs, then the rest, so LDS latency hides behind MFMAs.
        if constexpr (DT == MOE_BF16) {
          __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);
#pragma unroll
          for (int q = 0; q < 12; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, 40, 0);
        }
      } else if (mval > 0) {
#pragma unroll
        for (int fs = 0; fs < SL / 64; ++fs) {
          i32x4 fb[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            fb[j] = *reinterpret_cast<const i32x4*>(&lb[C::off(wn * 128 + j * 16 + row, fs * 4 + grp)]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i < mval) {
              const i32x4 fa = *reinterpret_cast<const i32x4*>(&la[C::off(wm * 64 + i * 16 + row, fs * 4 + grp)]);
#pragma unroll
              for (int j = 0; j < 8; ++j) F::mma(acc[i][j], fa, fb[j]);
            }
        }
      }
    } else {
      const float* sa_l = lds_s + st * (kTM + kTN);
      const float* sb_l = sa_l + kTM;
      // two halves of 4 column tiles keep the B fragments within the register budget
#pragma unroll
      for (int jh = 0; jh < 2; ++jh) {
        i32x4 fb0[4], fb1[4];
        float sb[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int n = wn * 128 + (4 * jh + jj) * 16 + row;
          fb0[jj] = *reinterpret_cast<const i32x4*>(&lb[C::off(n, grp)]);
          fb1[jj] = *reinterpret_cast<const i32x4*>(&lb[C::off(n, 4 + grp)]);
          sb[jj] = sb_l[n];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i < mval) {
            const int r = wm * 64 + i * 16 + row;
            const i32x4 fa0 = *reinterpret_cast<const i32x4*>(&la[C::off(r, grp)]);
            const i32x4 fa1 = *reinterpret_cast<const i32x4*>(&la[C::off(r, 4 + grp)]);
            float sa[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) sa[q] = sa_l[wm * 64 + i * 16 + 4 * grp + q];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const f32x4 p = F::mma128(fa0, fa1, fb0[jj], fb1[jj]);
#pragma unroll
              for (int q = 0; q < 4; ++q)
                acc[i][4 * jh + jj][q] = fmaf(p[q], sa[q] * sb[jj], acc[i][4 * jh + jj][q]);
            }
          }
        }
      }
    }
  }

  // ---- epilogue: lane holds rows wm*64 + i*16 + 4*grp + q, columns wn*128 + j*16 + row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= mval) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = wm * 64 + i * 16 + 4 * grp + q;
      if (r >= rows) continue;
      if (MODE == 1) {
        const size_t hrow = (size_t)(gr.slot0 + row0 + r) * a.I;
#pragma unroll
        for (int jp = 0; jp < 4; ++jp) {
          const float gv = acc[i][2 * jp][q], uv = acc[i][2 * jp + 1][q];
          const int col = nt * (kTN / 2) + (4 * wn + jp) * 16 + row;
          if (col < a.I) store_h<DT>(a.h, hrow + col, silu(gv) * uv);
        }
      } else {
        uint8_t* ybase = gr.routed ? a.y_sorted : a.y_shared;
        const size_t yrow = (size_t)(gr.routed ? gr.slot0 + row0 + r : row0 + r) * a.H;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = nt * kTN + wn * 128 + j * 16 + row;
          if (col < a.H) store_y<DT>(ybase, yrow + col, acc[i][j][q]);
        }
      }
    }
  }
}

template <int DT, int MODE>
hipError_t launch_fat(const char* name, int grid, int ntn, const Args& a, hipStream_t st) {
  constexpr bool FP8 = DT == MOE_FP8_E4M3;
  using C = TileCfg<DT>;
  const size_t smem = (size_t)C::NST * C::STAGE + (FP8 ? C::NST * (kTM + kTN) * sizeof(float) : 0);
  static bool attr_set = false;   // raise the dynamic-LDS limit once per process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_fat_kernel<DT, MODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  MOE_LAUNCH(name, (ffn_fat_kernel<DT, MODE>), dim3(grid), dim3(512), smem, st, a, ntn);
  return hipGetLastError();
}

// The shared expert: its own launches, on the stream it is given.
template <int DT>
hipError_t run_shared(const moe_cfg& c, Args a, hipStream_t st) {
  a.shared_only = 1;
  const int P = a.P;
  hipError_t e;
  for (int mode = 1; mode <= 2; ++mode) {
    if (mode == 2 && DT == MOE_FP8_E4M3) {   // its rows [P, P + T) of h
      e = moe::launch_quant_fp8(c.T, c.I, a.qb, a.h + (size_t)P * c.I * 4, MOE_F32,
                                const_cast<uint8_t*>(a.a2) + (size_t)P * c.I,
                                const_cast<float*>(a.a2s) + (size_t)P * (c.I / a.qb), st);
      if (e != hipSuccess) return e;
    }
    const int N = mode == 1 ? c.I : c.H;
    if (c.T <= kSkinnyRows) {
      const int sh_items = N / (mode == 1 ? 4 * kShNT : 8 * kShNT);
      const char* shn = mode == 1 ? "ffn_gemm1_shared_skinny" : "ffn_gemm2_shared_skinny";
#define MOE_SH_LAUNCH(M, MT) \
      MOE_LAUNCH(shn, (ffn_shared_skinny_kernel<DT, M, MT>), dim3(sh_items), dim3(64 * kShKS), 0, st, a)
      if (mode == 1) {
        if (c.T <= 8) MOE_SH_LAUNCH(1, 1); else if (c.T <= 16) MOE_SH_LAUNCH(1, 2); else MOE_SH_LAUNCH(1, 4);
      } else {
        if (c.T <= 8) MOE_SH_LAUNCH(2, 1); else if (c.T <= 16) MOE_SH_LAUNCH(2, 2); else MOE_SH_LAUNCH(2, 4);
      }
#undef MOE_SH_LAUNCH
      if ((e = hipGetLastError()) != hipSuccess) return e;
    } else {
      const int ntn = mode == 1 ? moe::ceil_div(c.I, kTN / 2) : moe::ceil_div(c.H, kTN);
      const int grid = moe::ceil_div(c.T, kTM) * ntn;
      e = mode == 1 ? launch_fat<DT, 1>("ffn_gemm1_shared_tiled", grid, ntn, a, st)
                    : launch_fat<DT, 2>("ffn_gemm2_shared_tiled", grid, ntn, a, st);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// The routed experts, on the stream it is given: plan, then per projection
// the three skinny classes and the tiled groups.
template <int DT>
hipError_t run_routed(const moe_cfg& c, Args a, hipStream_t st) {
  a.shared_only = 0;
  const int G = a.G;
  MOE_LAUNCH("ffn_plan", ffn_plan_kernel, dim3(1), dim3(512), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int P = a.P;
  // Upper bound of the fat tiles: a token picks k distinct experts, so a
  // routed group has at most T rows and none is fat when T <= kSkinnyRows.
  // Otherwise at most ceil(P / kTileRows) full tiles plus one partial tile per
  // fat group, and at most min(E, P / (kSkinnyRows + 1)) fat groups.
  const int fat_groups = c.T > kSkinnyRows ? (P / (kSkinnyRows + 1) < c.E ? P / (kSkinnyRows + 1) : c.E) : 0;
  const int max_fat = fat_groups > 0 ? moe::ceil_div(P, kTileRows) + fat_groups : 0;
  for (int mode = 1; mode <= 2; ++mode) {
    if (mode == 2 && DT == MOE_FP8_E4M3) {
      e = moe::launch_quant_fp8(P, c.I, a.qb, a.h, MOE_F32, const_cast<uint8_t*>(a.a2), const_cast<float*>(a.a2s), st);
      if (e != hipSuccess) return e;
    }
    const int N = mode == 1 ? c.I : c.H;
    // upper bounds of the three skinny lists: a group of class c has > 8 * 2^(c-1) rows
    int sk_groups[3];
    for (int cls = 0; cls < 3; ++cls) {
      const int min_rows = cls == 0 ? 1 : (4 << cls) + 1;   // 1, 9, 17
      const int bound = P / min_rows;
      sk_groups[cls] = bound < c.E ? bound : c.E;
    }
    const int ntn = mode == 1 ? moe::ceil_div(c.I, kTN / 2) : moe::ceil_div(c.H, kTN);
    const int fat_grid = max_fat * ntn;
    static const char* const kSkName[2][3] = {
        {"ffn_gemm1_skinny_m8", "ffn_gemm1_skinny_m16", "ffn_gemm1_skinny_m32"},
        {"ffn_gemm2_skinny_m8", "ffn_gemm2_skinny_m16", "ffn_gemm2_skinny_m32"}};
    const char* fatn = mode == 1 ? "ffn_gemm1_tiled" : "ffn_gemm2_tiled";
#define MOE_SK_LAUNCH(M, CLS)                                                                   \
    if (sk_groups[CLS] > 0) {                                                                   \
      MOE_LAUNCH(kSkName[M - 1][CLS], (ffn_skinny_kernel<DT, M, CLS>), dim3((moe::ceil_div((long long)sk_groups[CLS] * (N / ((M == 1 ? 4 : 8) * kSkNT)), 4) + 7) & ~7LL), \
                 dim3(256), 0, st, a);                                                          \
      if ((e = hipGetLastError()) != hipSuccess) return e;                                     \
    }
    if (mode == 1) {
      MOE_SK_LAUNCH(1, 0) MOE_SK_LAUNCH(1, 1) MOE_SK_LAUNCH(1, 2)
      if (fat_grid > 0 && (e = launch_fat<DT, 1>(fatn, fat_grid, ntn, a, st)) != hipSuccess) return e;
    } else {
      MOE_SK_LAUNCH(2, 0) MOE_SK_LAUNCH(2, 1) MOE_SK_LAUNCH(2, 2)
      if (fat_grid > 0 && (e = launch_fat<DT, 2>(fatn, fat_grid, ntn, a, st)) != hipSuccess) return e;
    }
#undef MOE_SK_LAUNCH
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// A tiled shared expert (T > kSkinnyRows) runs on a side stream forked from
// st (an event records st's position, the side stream waits on it) and
// joined back at the end (st waits on an event recorded after the shared
// launches), so it overlaps the routed experts: at a few hundred tokens its
// GEMMs have too few tiles to fill the device on their own.  It is enqueued
// first so that its large workgroups find free CUs before the routed kernels
// fill the device.  Both halves write disjoint rows of h and separate
// outputs.  A skinny shared expert stays on st: it streams weights like the
// routed skinny kernels, and running it beside them only adds contention.
template <int DT>
hipError_t run_ffn(const moe_cfg& c, const Args& a, hipStream_t st) {
  if (!a.has_shared) return run_routed<DT>(c, a, st);
  if (c.T <= kSkinnyRows) {
    hipError_t e = run_shared<DT>(c, a, st);
    return e != hipSuccess ? e : run_routed<DT>(c, a, st);
  }
  moe::SideStream side;
  hipError_t e = moe::side_stream(&side);
  if (e != hipSuccess) return e;
  if ((e = hipEventRecord(side.fork, st)) != hipSuccess) return e;
  if ((e = hipStreamWaitEvent(side.stream, side.fork, 0)) != hipSuccess) return e;
  hipError_t es = run_shared<DT>(c, a, side.stream);
  hipError_t er = es == hipSuccess ? run_routed<DT>(c, a, st) : hipSuccess;
  // join even after a failed launch, so that work queued later on st never
  // runs ahead of work already queued on the side stream
  if ((e = hipEventRecord(side.join, side.stream)) == hipSuccess) e = hipStreamWaitEvent(st, side.join, 0);
  return es != hipSuccess ? es : er != hipSuccess ? er : e;
}

}  // namespace

namespace moe {

size_t ffn_plan_ints(const moe_cfg& c) {
  const int P = c.T * c.k;
  const int G = c.E + (c.I_shared > 0 ? 1 : 0);
  const int max_fat = ceil_div(P, kTileRows) + c.E + (c.I_shared > 0 ? ceil_div(c.T, kTileRows) : 0);
  return kPlanHead + 3 * (size_t)G + 2 * (size_t)max_fat;
}

size_t ffn_h_elem_bytes(const moe_cfg& c) { return c.w_dtype == MOE_BF16 ? 2 : 4; }

hipError_t launch_expert_ffn(const moe_cfg& c, const void* x, const int32_t* offsets,
                             const int32_t* sorted_pair, const moe_weights& w, void* y_sorted,
                             void* y_shared, const FfnWs& ws, hipStream_t st) {
  Args a{};
  a.T = c.T;
  a.H = c.H;
  a.E = c.E;
  a.k = c.k;
  a.I = c.I;
  a.P = c.T * c.k;
  a.has_shared = c.I_shared > 0;
  a.qb = c.quant_block;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.w13 = static_cast<const uint8_t*>(w.w13);
  a.w13s = w.w13_scale;
  a.ws13 = static_cast<const uint8_t*>(w.ws13);
  a.ws13s = w.ws13_scale;
  a.w2 = static_cast<const uint8_t*>(w.w2);
  a.w2s = w.w2_scale;
  a.ws2 = static_cast<const uint8_t*>(w.ws2);
  a.ws2s = w.ws2_scale;
  a.h = static_cast<uint8_t*>(ws.h);
  a.y_sorted = static_cast<uint8_t*>(y_sorted);
  a.y_shared = static_cast<uint8_t*>(y_shared);
  a.plan = ws.plan;
  a.G = c.E + (a.has_shared ? 1 : 0);
  if (c.w_dtype == MOE_FP8_E4M3) {
    hipError_t e = launch_quant_fp8(c.T, c.H, c.quant_block, x, MOE_BF16, ws.xq, ws.xs, st);
    if (e != hipSuccess) return e;
    a.a1 = ws.xq;
    a.a1s = ws.xs;
    a.a2 = ws.hq;
    a.a2s = ws.hs;
    return run_ffn<MOE_FP8_E4M3>(c, a, st);
  }
  a.a1 = static_cast<const uint8_t*>(x);
  a.a2 = a.h;
  if (c.w_dtype == MOE_BF16) return run_ffn<MOE_BF16>(c, a, st);
  return run_ffn<MOE_F32>(c, a, st);
}

}  // namespace moe
