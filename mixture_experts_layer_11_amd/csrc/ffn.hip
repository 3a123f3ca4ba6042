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
constexpr int kBM = 128;         // fat tile rows
constexpr int kBN = 128;         // fat tile columns (GEMM1: 64 gate + 64 up)
constexpr int kSkNT = 4;         // skinny: 16-row weight tiles per wave

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
  float* y_sorted;
  float* y_shared;
  const int32_t* plan;          // [0] n_skinny, [1] n_fat, [2..2+G) skinny groups, then fat (group,row0)
  int G;
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

// ------------------------------------------------------------------ plan

__global__ __launch_bounds__(512) void ffn_plan_kernel(Args a) {
  __shared__ int sk[512];
  __shared__ int ft[512];
  const int g = threadIdx.x;
  int m = 0;
  if (g < a.G) m = g < a.E ? a.offsets[g + 1] - a.offsets[g] : a.T;
  const int is_sk = (m > 0 && m <= kSkinnyRows) ? 1 : 0;
  const int tiles = m > kSkinnyRows ? (m + kBM - 1) / kBM : 0;
  sk[g] = is_sk;
  ft[g] = tiles;
  __syncthreads();
  for (int d = 1; d < 512; d <<= 1) {
    const int v1 = g >= d ? sk[g - d] : 0;
    const int v2 = g >= d ? ft[g - d] : 0;
    __syncthreads();
    sk[g] += v1;
    ft[g] += v2;
    __syncthreads();
  }
  int32_t* plan = const_cast<int32_t*>(a.plan);
  if (g == 511) {
    plan[0] = sk[511];
    plan[1] = ft[511];
  }
  if (is_sk) plan[2 + sk[g] - 1] = g;
  const int t0 = ft[g] - tiles;
  int32_t* fat = plan + 2 + a.G;
  for (int i = 0; i < tiles; ++i) {
    fat[2 * (t0 + i)] = g;
    fat[2 * (t0 + i) + 1] = i * kBM;
  }
}

// ------------------------------------------------------------------ skinny grouped GEMM

// One wave = one work item: kSkNT weight tiles of 16 rows over the full K,
// against up to 32 activation rows (two 16-row M tiles).
template <int DT, int MODE>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(Args a) {
  using F = Frag<DT>;
  constexpr int NT = kSkNT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int cols_per_item = MODE == 1 ? 8 * NT : 16 * NT;   // h columns (mode 1) or y columns (mode 2)
  const int N = MODE == 1 ? a.I : a.H;
  const int items = N / cols_per_item;
  const int item = blockIdx.x * 4 + wave;
  const int gi = item / items;
  if (gi >= a.plan[0]) return;
  const int g = a.plan[2 + gi];
  const int it = item - gi * items;
  const Group gr = group_of(a, g);
  const int K = MODE == 1 ? a.H : a.I;
  const size_t krow = (size_t)K * F::ESZ;
  const int nmt = (gr.m + 15) >> 4;   // 1 or 2 (uniform)

  // A rows (this lane loads row `row` of each M tile)
  const uint8_t* pa[2];
  bool av[2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int r = mt * 16 + row;
    av[mt] = r < gr.m;
    int src = 0;
    if (av[mt]) src = MODE == 1 ? gemm1_src_row(a, gr, r) : gr.slot0 + r;
    pa[mt] = (MODE == 1 ? a.a1 : a.a2) + (size_t)src * krow + grp * 16;
  }
  // B rows (weight rows of the kSkNT tiles)
  const uint8_t* wbase;
  const float* wsbase = nullptr;
  if (MODE == 1) {
    wbase = gr.routed ? a.w13 + (size_t)g * 2 * a.I * krow : a.ws13;
    if (DT == MOE_FP8_E4M3) wsbase = gr.routed ? a.w13s + (size_t)g * 2 * a.I * (K / a.qb) : a.ws13s;
  } else {
    wbase = gr.routed ? a.w2 + (size_t)g * a.H * krow : a.ws2;
    if (DT == MOE_FP8_E4M3) wsbase = gr.routed ? a.w2s + (size_t)g * a.H * (K / a.qb) : a.ws2s;
  }
  int wrow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    if (MODE == 1) {
      const int c0 = it * cols_per_item;
      wrow[j] = (j < NT / 2 ? 0 : a.I) + c0 + 16 * (j % (NT / 2)) + row;
    } else {
      wrow[j] = it * cols_per_item + 16 * j + row;
    }
  }
  const uint8_t* pb[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) pb[j] = wbase + (size_t)wrow[j] * krow + grp * 16;

  f32x4 acc[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if constexpr (DT != MOE_FP8_E4M3) {
    const int nfrag = K / F::KF;
#pragma unroll 4
    for (int f = 0; f < nfrag; ++f) {
      const size_t off = (size_t)f * 64;
      i32x4 b[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) b[j] = ld16(pb[j] + off);
      const i32x4 a0 = av[0] ? ld16(pa[0] + off) : zero16();
#pragma unroll
      for (int j = 0; j < NT; ++j) F::mma(acc[0][j], a0, b[j]);
      if (nmt > 1) {
        const i32x4 a1 = av[1] ? ld16(pa[1] + off) : zero16();
#pragma unroll
        for (int j = 0; j < NT; ++j) F::mma(acc[1][j], a1, b[j]);
      }
    }
  } else {
    // Scales of the C rows this lane holds (rows 4*grp+i of each M tile) and of its B rows.
    const int nkb = K / a.qb;
    const float* sa_row[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + 4 * grp + i;
        int src = 0;
        if (r < gr.m) src = MODE == 1 ? gemm1_src_row(a, gr, r) : gr.slot0 + r;
        sa_row[mt][i] = (MODE == 1 ? a.a1s : a.a2s) + (size_t)src * nkb;
      }
    const float* sw_row[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) sw_row[j] = wsbase + (size_t)wrow[j] * nkb;
#pragma unroll 2
    for (int kb = 0; kb < nkb; ++kb) {
      const size_t off = (size_t)kb * 128;
      i32x4 b0[NT], b1[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        b0[j] = ld16(pb[j] + off);
        b1[j] = ld16(pb[j] + off + 64);
      }
      float sw[NT];
#pragma unroll
      for (int j = 0; j < NT; ++j) sw[j] = sw_row[j][kb];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        if (mt < nmt) {
          const i32x4 a0 = av[mt] ? ld16(pa[mt] + off) : zero16();
          const i32x4 a1 = av[mt] ? ld16(pa[mt] + off + 64) : zero16();
          float sa[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) sa[i] = sa_row[mt][i][kb];
#pragma unroll
          for (int j = 0; j < NT; ++j) {
            const f32x4 p = F::mma128(a0, a1, b0[j], b1[j]);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[mt][j][i] = fmaf(p[i], sa[i] * sw[j], acc[mt][j][i]);
          }
        }
      }
    }
  }

  // Epilogue: lane holds rows 4*grp+i of each M tile, column `row` of each N tile.
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    if (mt >= nmt) break;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = mt * 16 + 4 * grp + i;
      if (r >= gr.m) continue;
      if (MODE == 1) {
        const size_t hrow = (size_t)(gr.slot0 + r) * a.I;
#pragma unroll
        for (int j = 0; j < NT / 2; ++j) {
          const float gv = acc[mt][j][i], uv = acc[mt][j + NT / 2][i];
          const int col = it * cols_per_item + 16 * j + row;
          store_h<DT>(a.h, hrow + col, silu(gv) * uv);
        }
      } else {
        float* yrow = gr.routed ? a.y_sorted + (size_t)(gr.slot0 + r) * a.H : a.y_shared + (size_t)r * a.H;
#pragma unroll
        for (int j = 0; j < NT; ++j) yrow[it * cols_per_item + 16 * j + row] = acc[mt][j][i];
      }
    }
  }
}

// ------------------------------------------------------------------ fat grouped GEMM

// LDS tile: 128 rows x 128 bytes, 16-byte chunk c of row r stored at chunk c ^ (r & 7).
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

template <int DT, int MODE>
__global__ __launch_bounds__(256) void ffn_fat_kernel(Args a, int ntn) {
  using F = Frag<DT>;
  constexpr bool FP8 = DT == MOE_FP8_E4M3;
  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][kBM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][kBN * 128];
  __shared__ float lds_sa[2][FP8 ? kBM : 1];
  __shared__ float lds_sb[2][FP8 ? kBN : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int tile = blockIdx.x / ntn;
  const int nt = blockIdx.x - tile * ntn;
  if (tile >= a.plan[1]) return;
  const int32_t* fat = a.plan + 2 + a.G;
  const int g = fat[2 * tile];
  const int row0 = fat[2 * tile + 1];
  const Group gr = group_of(a, g);
  const int rows = min(kBM, gr.m - row0);
  const int K = MODE == 1 ? a.H : a.I;
  const size_t krow = (size_t)K * F::ESZ;
  const int nkt = (int)(krow / 128);          // 128-byte K slices
  const int nkb = FP8 ? K / a.qb : 0;

  // ---- global source rows for this thread's 4 A chunks and 4 B chunks
  const int lc = tid & 7;          // 16-byte chunk within the 128-byte slice
  const int lr = tid >> 3;         // base row 0..31; rows lr + 32*i
  const uint8_t* ga[4];
  const uint8_t* gb[4];
  const uint8_t* asrc = MODE == 1 ? a.a1 : a.a2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = lr + 32 * i;
    const int rr = r < rows ? r : rows - 1;      // clamp: padded rows recompute a valid row, never stored
    const int src = MODE == 1 ? gemm1_src_row(a, gr, row0 + rr) : gr.slot0 + row0 + rr;
    ga[i] = asrc + (size_t)src * krow + lc * 16;
  }
  const uint8_t* wbase;
  const float* wsbase = nullptr;
  if (MODE == 1) {
    wbase = gr.routed ? a.w13 + (size_t)g * 2 * a.I * krow : a.ws13;
    if (FP8) wsbase = gr.routed ? a.w13s + (size_t)g * 2 * a.I * nkb : a.ws13s;
  } else {
    wbase = gr.routed ? a.w2 + (size_t)g * a.H * krow : a.ws2;
    if (FP8) wsbase = gr.routed ? a.w2s + (size_t)g * a.H * nkb : a.ws2s;
  }
  auto b_wrow = [&](int n) -> int {   // weight row of LDS B row n
    if (MODE == 1) {
      const int blk = n >> 4;          // 16-row block: even = gate, odd = up
      return ((blk & 1) ? a.I : 0) + nt * (kBN / 2) + (blk >> 1) * 16 + (n & 15);
    }
    return nt * kBN + n;
  };
#pragma unroll
  for (int i = 0; i < 4; ++i) gb[i] = wbase + (size_t)b_wrow(lr + 32 * i) * krow + lc * 16;

  // fp8 scale sources: thread tid < 128 loads A-row scale tid, 128..255 B-row scale tid-128
  const float* gs = nullptr;
  if constexpr (FP8) {
    if (tid < kBM) {
      const int r = tid < rows ? tid : rows - 1;
      const int src = MODE == 1 ? gemm1_src_row(a, gr, row0 + r) : gr.slot0 + row0 + r;
      gs = (MODE == 1 ? a.a1s : a.a2s) + (size_t)src * nkb;
    } else {
      gs = wsbase + (size_t)b_wrow(tid - kBM) * nkb;
    }
  }

  i32x4 ra[4], rb[4];
  float rs = 0.f;
  auto gload = [&](int kt) {
    const size_t off = (size_t)kt * 128;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(ga[i] + off);
      rb[i] = ld16(gb[i] + off);
    }
    if constexpr (FP8) rs = gs[kt];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lr + 32 * i;
      *reinterpret_cast<i32x4*>(&lds_a[buf][lds_off(r, lc)]) = ra[i];
      *reinterpret_cast<i32x4*>(&lds_b[buf][lds_off(r, lc)]) = rb[i];
    }
    if constexpr (FP8) {
      if (tid < kBM) lds_sa[buf][tid] = rs;
      else lds_sb[buf][tid - kBM] = rs;
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kt + 1);
    const uint8_t* la = lds_a[buf];
    const uint8_t* lb = lds_b[buf];
    if constexpr (!FP8) {
#pragma unroll
      for (int fs = 0; fs < 2; ++fs) {
        i32x4 fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const i32x4*>(&la[lds_off(wm * 64 + i * 16 + row, fs * 4 + grp)]);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = *reinterpret_cast<const i32x4*>(&lb[lds_off(wn * 64 + j * 16 + row, fs * 4 + grp)]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) F::mma(acc[i][j], fa[i], fb[j]);
      }
    } else {
      i32x4 fa0[4], fa1[4], fb0[4], fb1[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + row;
        fa0[i] = *reinterpret_cast<const i32x4*>(&la[lds_off(r, grp)]);
        fa1[i] = *reinterpret_cast<const i32x4*>(&la[lds_off(r, 4 + grp)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = wn * 64 + j * 16 + row;
        fb0[j] = *reinterpret_cast<const i32x4*>(&lb[lds_off(n, grp)]);
        fb1[j] = *reinterpret_cast<const i32x4*>(&lb[lds_off(n, 4 + grp)]);
      }
      float sa[4][4], sb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) sa[i][q] = lds_sa[buf][wm * 64 + i * 16 + 4 * grp + q];
#pragma unroll
      for (int j = 0; j < 4; ++j) sb[j] = lds_sb[buf][wn * 64 + j * 16 + row];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 p = F::mma128(fa0[i], fa1[i], fb0[j], fb1[j]);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(p[q], sa[i][q] * sb[j], acc[i][j][q]);
        }
    }
    if (kt + 1 < nkt) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows wm*64 + i*16 + 4*grp + q, columns wn*64 + j*16 + row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = wm * 64 + i * 16 + 4 * grp + q;
      if (r >= rows) continue;
      if (MODE == 1) {
        const size_t hrow = (size_t)(gr.slot0 + row0 + r) * a.I;
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
          const float gv = acc[i][2 * jp][q], uv = acc[i][2 * jp + 1][q];
          const int col = nt * (kBN / 2) + (2 * wn + jp) * 16 + row;
          store_h<DT>(a.h, hrow + col, silu(gv) * uv);
        }
      } else {
        float* yrow = gr.routed ? a.y_sorted + (size_t)(gr.slot0 + row0 + r) * a.H
                                : a.y_shared + (size_t)(row0 + r) * a.H;
#pragma unroll
        for (int j = 0; j < 4; ++j) yrow[nt * kBN + wn * 64 + j * 16 + row] = acc[i][j][q];
      }
    }
  }
}

template <int DT>
hipError_t run_ffn(const moe_cfg& c, Args a, hipStream_t st) {
  const int G = a.G;
  MOE_LAUNCH("ffn_plan", ffn_plan_kernel, dim3(1), dim3(512), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int P = a.P;
  const int max_fat = moe::ceil_div(P, kBM) + (P / (kSkinnyRows + 1) < c.E ? P / (kSkinnyRows + 1) : c.E) +
                      (a.has_shared ? moe::ceil_div(c.T, kBM) : 0);
  for (int mode = 1; mode <= 2; ++mode) {
    if (mode == 2 && DT == MOE_FP8_E4M3) {
      e = moe::launch_quant_fp8(P + (a.has_shared ? c.T : 0), c.I, a.qb, a.h, MOE_F32,
                                const_cast<uint8_t*>(a.a2), const_cast<float*>(a.a2s), st);
      if (e != hipSuccess) return e;
    }
    const int N = mode == 1 ? c.I : c.H;
    const int sk_items = N / (mode == 1 ? 8 * kSkNT : 16 * kSkNT);
    const int sk_grid = moe::ceil_div((long long)G * sk_items, 4);
    const int ntn = mode == 1 ? c.I / (kBN / 2) : c.H / kBN;
    const int fat_grid = max_fat * ntn;
    if (mode == 1) {
      MOE_LAUNCH("ffn_gemm1_skinny", (ffn_skinny_kernel<DT, 1>), dim3(sk_grid), dim3(256), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (fat_grid > 0) MOE_LAUNCH("ffn_gemm1_tiled", (ffn_fat_kernel<DT, 1>), dim3(fat_grid), dim3(256), 0, st, a, ntn);
    } else {
      MOE_LAUNCH("ffn_gemm2_skinny", (ffn_skinny_kernel<DT, 2>), dim3(sk_grid), dim3(256), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      if (fat_grid > 0) MOE_LAUNCH("ffn_gemm2_tiled", (ffn_fat_kernel<DT, 2>), dim3(fat_grid), dim3(256), 0, st, a, ntn);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

namespace moe {

size_t ffn_plan_ints(const moe_cfg& c) {
  const int P = c.T * c.k;
  const int G = c.E + (c.I_shared > 0 ? 1 : 0);
  const int max_fat = ceil_div(P, kBM) + c.E + (c.I_shared > 0 ? ceil_div(c.T, kBM) : 0);
  return 2 + (size_t)G + 2 * (size_t)max_fat;
}

size_t ffn_h_elem_bytes(const moe_cfg& c) { return c.w_dtype == MOE_BF16 ? 2 : 4; }

hipError_t launch_expert_ffn(const moe_cfg& c, const void* x, const int32_t* offsets,
                             const int32_t* sorted_pair, const moe_weights& w, float* y_sorted,
                             float* y_shared, const FfnWs& ws, hipStream_t st) {
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
  a.y_sorted = y_sorted;
  a.y_shared = y_shared;
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
