// Skinny grouped GEMM: expert groups of 1..32 rows (decode), streamed.
//
// Perplexity's "Lower latency and higher throughput with multi-node DeepSeek
// deployment" (section "GroupGEMM") finds the grouped GEMM bandwidth-bound
// while the rows per expert are few; here each weight byte is read from HBM
// exactly once, in whole 128-byte cache lines, against the group's rows.
//
// Routed groups stream through a per-wave LDS ring (skinny_ring below).  The
// decode shared expert of 17..32 tokens streams straight into registers
// (skinny_pass), with this layout: one wave load instruction covers 8 weight
// rows x one 128-byte window: lane l reads row (l % 8), 16-byte chunk c(l) =
// 4 * ((l >> 3) & 1) + (l >> 4).  Fed as the B operand of a 16x16 MFMA,
// column n (lane l % 16) thus holds weight row n % 8, and columns n and n + 8
// hold the two complementary 64-byte halves of the window.  The A operand
// mirrors this: M row m holds token m % 8 with the same chunk rule.  The
// diagonal 8x8 blocks of the 16x16 result are then the two K halves of the
// same (token, row) dot products and the off-diagonal blocks are discarded:
// out[t][r] = C[t][r] + C[t+8][r+8], which sits in lanes L and L ^ 40.

#include "ffn.h"

namespace {

using namespace moe::ffn;

// Weights are read exactly once: nontemporal loads keep them from displacing
// the reused activation rows in the caches.
__device__ __forceinline__ i32x4 ldw16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(p));
}

__device__ __forceinline__ int sk_chunk(int lane) { return 4 * ((lane >> 3) & 1) + (lane >> 4); }

// Fold the two K halves and store: lanes L = 16*h + r (h < 2, r < 8) end up
// holding tokens 4*h + i (i = 0..3) of each M tile for weight row r of each
// tile.  GEMM1 applies SwiGLU to the gate/up tile pairs.
template <int DT, int MODE, int MT, int NT, int NTP>
__device__ __forceinline__ void skinny_epilogue(const Args& a, const Group& gr, int it, int p, int lane,
                                                f32x4 (&acc)[MT][NTP]) {
  const int r8 = lane & 7;
  const int cols_per_item = MODE == 1 ? 4 * NT : 8 * NT;   // h columns (GEMM1) or y columns (GEMM2)
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
          store_h<DT>(a.h, hrow + it * cols_per_item + 8 * (p * (NTP / 2) + j) + r8, silu_for<DT>(gv) * uv);
        }
      } else {
        uint8_t* ybase = gr.routed ? a.y_sorted : a.y_shared;
        const size_t yrow = (size_t)out_row(a, gr, r) * a.H;
#pragma unroll
        for (int j = 0; j < NTP; ++j) store_y<DT>(ybase, yrow + it * cols_per_item + 8 * (p * NTP + j) + r8, acc[mt][j][i]);
      }
    }
  }
}

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
    if (FP8) wsbase = gr.routed ? a.w13s + (size_t)g * ((2 * a.I) >> a.wsr_shift) * nwin : a.ws13s;
  } else {
    wbase = gr.routed ? a.w2 + (size_t)g * a.H * krow : a.ws2;
    if (FP8) wsbase = gr.routed ? a.w2s + (size_t)g * (a.H >> a.wsr_shift) * nwin : a.ws2s;
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
        for (int j = 0; j < NTP; ++j) sw[u][j] = wsbase[(size_t)(wrow[j] >> a.wsr_shift) * nwin + wu];
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

  skinny_epilogue<DT, MODE, MT, NT, NTP>(a, gr, it, p, lane, acc);
}

// Streaming through a per-wave LDS ring.  Each K window of the item (the NT
// weight tiles' and MT activation tiles' 8-row x 128-byte blocks, plus for
// fp8 the window's weight and activation scales) goes global -> LDS directly
// into slot w % D of the wave's ring, and the wave issues window w + D as
// soon as it has read window w back into registers, so D windows are always
// in flight: the wave's own queue, not other waves, hides the HBM latency,
// and the wide items can use most of the register file.  Only this wave
// touches its ring, so the waits are vmcnt waits and there are no barriers.
//
// Each direct load reads 8 whole rows x 128 bytes (lane L: row L / 8, chunk
// (L % 8) ^ (L / 8)), stored row-major with 16-byte chunk c of row r at chunk
// c ^ r.  Read back, 16 rows (two blocks) form one operand of a full 16x16
// MFMA tile: activation rows along M, weight rows along N; 8 lanes reading
// the same chunk of 8 rows hit 8 distinct 16-byte slots, free of bank
// conflicts.  The 8-row class pairs its M tile with itself (the upper 8 C
// rows are discarded).  bf16/fp32 take the window as two K steps (chunks
// 4s + g for lane group g), fp8 as one 16x16x128 step (chunks g and g + 4).
//
// fp8 scales of a window: lane L fetches the weight scale of item row L
// (tile L / 8, row L % 8) and, for L < 32, the activation scale of group row
// L; a lane's C values then need the weight scale of its column and the
// activation scales of 4 consecutive rows per M pair.
template <int DT, int MT, int NT, int D> struct RingCfg {
  static constexpr bool FP8 = DT == MOE_FP8_E4M3;
  static constexpr int NB = NT + MT;                   // 1 KB blocks (direct loads) per window
  static constexpr int WIN = NB * 1024;                // LDS bytes per ring slot
  // fp8 4-window scale blocks: the windows in flight (D + 1) span at most
  // (D + 3) / 4 + 1 blocks, each 2 KB (weight then activation scales); the
  // per-window path takes 512 bytes per ring slot
  static constexpr int SBUF = (D + 3) / 4 + 1;
  static constexpr int SCL = FP8 ? (SBUF * 2048 > D * 512 ? SBUF * 2048 : D * 512) : 0;   // after the D slots
  static constexpr int WAVE_BYTES = D * WIN + SCL;     // one wave's LDS
  static constexpr int MP = MT > 1 ? MT / 2 : 1;       // 16-row M pairs
  static constexpr int NP = NT / 2;                    // 16-row N pairs
};

template <int DT, int MODE, int MT, int NT, int D>
__device__ __forceinline__ void skinny_ring(const Args& a, const Group& gr, int g, int it, int lane, uint8_t* ring) {
  using F = Frag<DT>;
  using R = RingCfg<DT, MT, NT, D>;
  constexpr bool FP8 = R::FP8;
  constexpr int MP = R::MP, NP = R::NP;
  static_assert(NT % 2 == 0 && (MODE == 2 || NT % 4 == 0), "GEMM1 pairs gate and up 16-row blocks");
  const int cols_per_item = MODE == 1 ? 4 * NT : 8 * NT;
  const int K = MODE == 1 ? a.H : a.I;
  const size_t krow = (size_t)K * F::ESZ;
  const int nwin = (int)(krow / 128);

  const uint8_t* abase = MODE == 1 ? a.a1 : a.a2;
  const uint8_t* wbase;
  const float* wsbase = nullptr;
  if (MODE == 1) {
    wbase = gr.routed ? a.w13 + (size_t)g * 2 * a.I * krow : a.ws13;
    if (FP8) wsbase = gr.routed ? a.w13s + (size_t)g * ((2 * a.I) >> a.wsr_shift) * nwin : a.ws13s;
  } else {
    wbase = gr.routed ? a.w2 + (size_t)g * a.H * krow : a.ws2;
    if (FP8) wsbase = gr.routed ? a.w2s + (size_t)g * (a.H >> a.wsr_shift) * nwin : a.ws2s;
  }
  // weight row of tile j, row r (GEMM1: first half gate tiles, second half the matching up tiles)
  auto wrow_of = [&](int j, int r) -> int {
    return MODE == 1 ? (j < NT / 2 ? 0 : a.I) + it * cols_per_item + 8 * (j % (NT / 2)) + r
                     : it * cols_per_item + 8 * j + r;
  };
  // token row (GEMM1) or h row (GEMM2) of group row r, clamped: clamped rows feed C rows never stored
  auto src_row = [&](int r) -> int {
    r = min(r, gr.m - 1);
    return MODE == 1 ? gemm1_src_row(a, gr, r) : gr.slot0 + r;
  };
  // this lane's direct-load slot: row lr of each block, global chunk lc (stored at chunk lane % 8)
  const int lr = lane >> 3, lc = (lane & 7) ^ lr;
  const uint8_t* pb0 = wbase + (size_t)wrow_of(0, lr) * krow + lc * 16;
  size_t tile_off[NT];   // tile j sits a wave-uniform distance from tile 0
#pragma unroll
  for (int j = 0; j < NT; ++j) tile_off[j] = (size_t)(wrow_of(j, 0) - wrow_of(0, 0)) * krow;
  const uint8_t* pa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) pa[mt] = abase + (size_t)src_row(mt * 8 + lr) * krow + lc * 16;
  const float* psw = nullptr;
  const float* psa = nullptr;
  if constexpr (FP8) {
    psw = wsbase + (size_t)(wrow_of(lane >> 3, lane & 7) >> a.wsr_shift) * nwin;
    psa = (MODE == 1 ? a.a1s : a.a2s) + (size_t)src_row(lane & 31) * nwin;
  }

  // fp8 scales: when nwin % 4 == 0 (K a multiple of 512), one 16-byte load
  // per lane fetches 4 windows' scales of its row, into one of SBUF 2 KB
  // blocks (weight scales, then activation scales) of the scale area: each
  // scale row's cache line is touched once per 4 windows, not every window
  // (a window's 64 weight scales lie in 64 different rows and lines).  Else
  // each window's scales go, 4 bytes per lane, into a 512-byte slot per ring
  // slot.
  uint8_t* scl = ring + D * R::WIN;
  const bool blk4 = FP8 && (nwin & 3) == 0;
  auto loads_of = [&](int w) -> int {   // direct loads of window w
    return R::NB + (FP8 ? (blk4 ? ((w & 3) == 0 ? 2 : 0) : 2) : 0);
  };
  // The item's K windows are taken in the rotated order w0, w0 + 1, ..,
  // nwin - 1, 0, .., w0 - 1 (w below counts steps; window (w + w0) % nwin is
  // read).  With rows a power of two bytes long, every row's window w sits at
  // the same address modulo the row length, and waves that all start at
  // window 0 crowd the same HBM channels: a start that differs from item to
  // item spreads them (4 KB rows: 6.0 -> 7.1 TB/s in a read-only probe of
  // this access pattern; decode16's GEMM2 397 -> 375 us).  fp8 keeps the
  // plain order: its 2 KB GEMM2 rows measured 1% slower rotated (by whole
  // 4-window scale blocks, which the blocked scales need).
  const int w0 = !FP8 && (krow & (krow - 1)) == 0 ? (g * 7 + it * 5) % nwin : 0;
  auto issue = [&](int sl, int w) {
    uint8_t* base = ring + sl * R::WIN;
    const int wa = w + w0 < nwin ? w + w0 : w + w0 - nwin;   // the window read at step w
    const size_t off = (size_t)wa * 128;
#pragma unroll
    for (int j = 0; j < NT; ++j) __builtin_amdgcn_global_load_lds(pb0 + (tile_off[j] + off), base + j * 1024, 16, 0, 2);   // nt
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) __builtin_amdgcn_global_load_lds(pa[mt] + off, base + (NT + mt) * 1024, 16, 0, 0);
    if constexpr (FP8) {
      if (blk4) {
        if ((w & 3) == 0) {
          uint8_t* sbk = scl + ((w >> 2) % R::SBUF) * 2048;
          __builtin_amdgcn_global_load_lds(psw + wa, sbk, 16, 0, 0);
          __builtin_amdgcn_global_load_lds(psa + wa, sbk + 1024, 16, 0, 0);
        }
      } else {
        __builtin_amdgcn_global_load_lds(psw + wa, scl + sl * 512, 4, 0, 0);
        __builtin_amdgcn_global_load_lds(psa + wa, scl + sl * 512 + 256, 4, 0, 0);
      }
    }
  };

  // operand reads: row n (0..15) of the 16-row pair starting at block blk0, logical chunk c
  const int n16 = lane & 15, grp = lane >> 4;
  const int rsw = (n16 & 7) * 128;
  auto frag = [&](const uint8_t* base, int blk, int c) -> i32x4 {
    return *reinterpret_cast<const i32x4*>(base + blk * 1024 + rsw + (((c ^ n16) & 7) << 4));
  };

  f32x4 acc[MP][NP];
#pragma unroll
  for (int mp = 0; mp < MP; ++mp)
#pragma unroll
    for (int np = 0; np < NP; ++np) acc[mp][np] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int sl, int w) {
    const uint8_t* base = ring + sl * R::WIN;
    const int ablk = NT + min(n16 >> 3, MT - 1);   // 8-row class: rows 8..15 repeat rows 0..7
    const int bblk = n16 >> 3;
    if constexpr (!FP8) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        i32x4 fa[MP], fb[NP];
#pragma unroll
        for (int mp = 0; mp < MP; ++mp) fa[mp] = frag(base, ablk + 2 * mp, 4 * s + grp);
#pragma unroll
        for (int np = 0; np < NP; ++np) fb[np] = frag(base, bblk + 2 * np, 4 * s + grp);
#pragma unroll
        for (int mp = 0; mp < MP; ++mp)
#pragma unroll
          for (int np = 0; np < NP; ++np) F::mma(acc[mp][np], fa[mp], fb[np]);
      }
    } else {
      i32x4 fa0[MP], fa1[MP], fb0[NP], fb1[NP];
      float sw[NP];
      f32x4 sa[MP];
      // C rows 4 * grp + i of M pair mp (the 8-row class repeats its 8 rows); column n16 of N pair np
      auto srow = [&](int mp, int i) -> int { return MT > 1 ? 16 * mp + 4 * grp + i : (4 * grp + i) & 7; };
      if (blk4) {   // [row][4 windows] floats: weight scales, then activation scales
        const float* sbk = reinterpret_cast<const float*>(scl + ((w >> 2) % R::SBUF) * 2048);
        const int wi = w & 3;
#pragma unroll
        for (int mp = 0; mp < MP; ++mp)
#pragma unroll
          for (int i = 0; i < 4; ++i) sa[mp][i] = sbk[256 + srow(mp, i) * 4 + wi];
#pragma unroll
        for (int np = 0; np < NP; ++np) sw[np] = sbk[(16 * np + n16) * 4 + wi];
      } else {
        const float* sb = reinterpret_cast<const float*>(scl + sl * 512);
#pragma unroll
        for (int mp = 0; mp < MP; ++mp) sa[mp] = *reinterpret_cast<const f32x4*>(sb + 64 + srow(mp, 0));
#pragma unroll
        for (int np = 0; np < NP; ++np) sw[np] = sb[16 * np + n16];
      }
#pragma unroll
      for (int mp = 0; mp < MP; ++mp) {
        fa0[mp] = frag(base, ablk + 2 * mp, grp);
        fa1[mp] = frag(base, ablk + 2 * mp, grp + 4);
      }
#pragma unroll
      for (int np = 0; np < NP; ++np) {
        fb0[np] = frag(base, bblk + 2 * np, grp);
        fb1[np] = frag(base, bblk + 2 * np, grp + 4);
      }
#pragma unroll
      for (int mp = 0; mp < MP; ++mp)
#pragma unroll
        for (int np = 0; np < NP; ++np) {
          const f32x4 pr = F::mma128(fa0[mp], fa1[mp], fb0[np], fb1[np]);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mp][np][i] = fmaf(pr[i], sa[mp][i] * sw[np], acc[mp][np][i]);
        }
    }
  };

#pragma unroll
  for (int d = 0; d < D; ++d)
    if (d < nwin) issue(d, d);
  static_assert((D - 1) * (R::NB + 2) < 64, "vmcnt counts of the later windows");
  int w = 0, slot = 0;
  // windows w + 1 .. w + D - 1 (those issued) stay in flight while w is consumed
  for (; w < nwin; ++w) {
    int later = 0;
#pragma unroll
    for (int d = 1; d < D; ++d)
      if (w + d < nwin) later += loads_of(w + d);
    if (FP8) wait_vmcnt_dyn(later);
    else if (w + D - 1 < nwin) wait_vmcnt<(D - 1) * R::NB>();
    else wait_vmcnt_dyn(later);
    compute(slot, w);
    if (w + D < nwin) {
      wait_lgkm0();   // the slot's reads are done before its refill can land
      issue(slot, w + D);
    }
    slot = slot + 1 == D ? 0 : slot + 1;
  }

  // epilogue: lane holds C rows 4 * grp + i of each M pair, column n16 of each N pair
#pragma unroll
  for (int mp = 0; mp < MP; ++mp) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mp + 4 * grp + i;
      if (r >= gr.m || r >= 8 * MT) continue;
      if (MODE == 1) {
        const size_t hrow = (size_t)(gr.slot0 + r) * a.I;
#pragma unroll
        for (int np = 0; np < NP / 2; ++np)   // gate pair np, up pair np + NP / 2
          store_h<DT>(a.h, hrow + it * cols_per_item + 16 * np + n16,
                      silu_for<DT>(acc[mp][np][i]) * acc[mp][np + NP / 2][i]);
      } else {
        uint8_t* ybase = gr.routed ? a.y_sorted : a.y_shared;
        const size_t yrow = (size_t)out_row(a, gr, r) * a.H;
#pragma unroll
        for (int np = 0; np < NP; ++np) store_y<DT>(ybase, yrow + it * cols_per_item + 16 * np + n16, acc[mp][np][i]);
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
// One wave = one work item (group, column block of sk_nt weight tiles) in a
// single pass over K through its LDS ring; waves past the class's list exit
// at once.  Every class uses the same items: an activation block then serves
// 4 or 8 weight tiles, which keeps the activation re-reads (one per item) a
// small share of the loads even at 32 rows.  The ring (3 windows x 9..12.5
// KB per wave for 8-tile items, 4..6 windows x 5..8 KB for 4-tile ones)
// takes 108..152 KB per workgroup: one workgroup per CU, one wave per SIMD.
constexpr int kRingDepth = 3;   // K windows in flight per wave (8-tile items)
constexpr size_t sk_ring_bytes(int wave_bytes) { return (size_t)4 * wave_bytes; }   // 4 waves
// Windows in flight for class MT: 4-tile items have smaller windows and run
// deeper rings, so a wave keeps about as many bytes in flight.
constexpr int ring_depth(int nt, int mt) { return nt >= 8 ? kRingDepth : (mt == 1 ? 6 : mt == 2 ? 5 : 4); }
// A wave's share of the LDS: the largest ring of the three classes.
template <int DT, int NT> constexpr int ring_wave_bytes() {
  constexpr int b1 = RingCfg<DT, 1, NT, ring_depth(NT, 1)>::WAVE_BYTES;
  constexpr int b2 = RingCfg<DT, 2, NT, ring_depth(NT, 2)>::WAVE_BYTES;
  constexpr int b4 = RingCfg<DT, 4, NT, ring_depth(NT, 4)>::WAVE_BYTES;
  return b1 > b2 ? (b1 > b4 ? b1 : b4) : (b2 > b4 ? b2 : b4);
}

template <int DT, int MODE>
__global__ __launch_bounds__(256) void ffn_skinny_kernel(Args a) {
  constexpr int NT = sk_nt(DT, MODE);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cols_per_item = MODE == 1 ? 4 * NT : 8 * NT;
  const int items = (MODE == 1 ? a.I : a.H) / cols_per_item;
  int local = blockIdx.x >> 3, cls = 2, n = 0, per_xcd = 0;
  for (; cls >= 0; --cls) {
    n = a.plan[cls] * items;                  // items of this class
    per_xcd = (((n + 3) >> 2) + 7) >> 3;      // its workgroups per XCD
    if (local < per_xcd) break;
    local -= per_xcd;
  }
  if (cls < 0) return;
  const int item = ((blockIdx.x & 7) * per_xcd + local) * 4 + wave;
  if (item >= n) return;
  const int gi = item / items, it = item - gi * items;
  int g;
  const Group gr = group_of_entry(a, a.plan[kPlanHead + cls * 2 * a.G + gi], &g);
  extern __shared__ __attribute__((aligned(16))) uint8_t sk_ring[];
  uint8_t* ring = sk_ring + wave * ring_wave_bytes<DT, NT>();
  if (cls == 2) skinny_ring<DT, MODE, 4, NT, ring_depth(NT, 4)>(a, gr, g, it, lane, ring);
  else if (cls == 1) skinny_ring<DT, MODE, 2, NT, ring_depth(NT, 2)>(a, gr, g, it, lane, ring);
  else skinny_ring<DT, MODE, 1, NT, ring_depth(NT, 1)>(a, gr, g, it, lane, ring);
}

// The shared expert when T <= kSkinnyRows: its row count is known on the
// host, so its launch is sized exactly, with narrow items (kShNT tiles) and
// the K range split over the kShKS waves of each workgroup.

template <int DT, int MODE, int MT>
__global__ __launch_bounds__(64 * kShKS) void ffn_shared_skinny_kernel(Args a) {
  constexpr int NTP = MT == 1 ? kShNT : (kShNT / MT >= 2 ? kShNT / MT : 2);
  __shared__ f32x4 red[(kShKS - 1) * MT * NTP * 64];
  const int lane = threadIdx.x & 63, ks = threadIdx.x >> 6;
  const Group gr = group_of(a, a.E);
  skinny_tile<DT, MODE, MT, kShNT, kShKS>(a, gr, a.E, blockIdx.x, lane, ks, red);
}

template <int DT, int MODE>
hipError_t launch_sk(unsigned grid, const Args& a, hipStream_t st) {
  constexpr size_t lds = sk_ring_bytes(ring_wave_bytes<DT, sk_nt(DT, MODE)>());
  static_assert(lds <= 160 * 1024, "LDS budget");
  hipError_t e = moe::ensure_dynamic_lds(reinterpret_cast<const void*>(&ffn_skinny_kernel<DT, MODE>), (int)lds);
  if (e != hipSuccess) return e;
  MOE_LAUNCH(MODE == 1 ? "ffn_gemm1_skinny" : "ffn_gemm2_skinny", (ffn_skinny_kernel<DT, MODE>), dim3(grid), dim3(256),
             lds, st, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_shared_skinny_t(int mode, int T, const Args& a, hipStream_t st) {
  const int N = mode == 1 ? a.I : a.H;
  const dim3 grid(N / (mode == 1 ? 4 * kShNT : 8 * kShNT));
  const char* name = mode == 1 ? "ffn_gemm1_shared_skinny" : "ffn_gemm2_shared_skinny";
#define MOE_SH(M, MT) MOE_LAUNCH(name, (ffn_shared_skinny_kernel<DT, M, MT>), grid, dim3(64 * kShKS), 0, st, a)
  if (mode == 1) {
    if (T <= 8) MOE_SH(1, 1); else if (T <= 16) MOE_SH(1, 2); else MOE_SH(1, 4);
  } else {
    if (T <= 8) MOE_SH(2, 1); else if (T <= 16) MOE_SH(2, 2); else MOE_SH(2, 4);
  }
#undef MOE_SH
  return hipGetLastError();
}

}  // namespace

namespace moe {
namespace ffn {

template <int DT>
hipError_t launch_skinny(int mode, unsigned grid, const Args& a, hipStream_t st) {
  return mode == 1 ? launch_sk<DT, 1>(grid, a, st) : launch_sk<DT, 2>(grid, a, st);
}
template <int DT>
hipError_t launch_shared_skinny(int mode, int T, const Args& a, hipStream_t st) {
  return launch_shared_skinny_t<DT>(mode, T, a, st);
}

#define MOE_INST(DT)                                                                                \
  template hipError_t launch_skinny<DT>(int, unsigned, const Args&, hipStream_t);                   \
  template hipError_t launch_shared_skinny<DT>(int, int, const Args&, hipStream_t);
MOE_INST(MOE_F32)
MOE_INST(MOE_BF16)
MOE_INST(MOE_FP8_E4M3)
#undef MOE_INST

}  // namespace ffn
}  // namespace moe
