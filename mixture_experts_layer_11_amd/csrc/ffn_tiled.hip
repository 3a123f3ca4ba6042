// Tiled grouped GEMM: expert groups of more than 32 rows (prefill), and the
// shared expert beyond 32 tokens, on MFMA tiles with LDS-staged operands.
//
// Perplexity's "Lower latency and higher throughput with multi-node DeepSeek
// deployment" (sections "GroupGEMM" and "Future work") finds the grouped
// GEMM compute-bound once the rows per expert are many.

#include <type_traits>

#include "ffn.h"

namespace {

using namespace moe::ffn;

// Output tiles of TM x TN per workgroup of 8 waves, with 16x16 MFMAs:
//   TM = 256: 4 waves along M x 2 along N, 64 x 128 each, 2 LDS stages
//             (groups of 256 rows and more: the prefill regime; fp8: the
//             last 129..255 rows of a group);
//   TM = 256, TN = 128 (the fp8 shared expert's GEMM1): 64 x 64 per wave,
//             3 LDS stages;
//   TM = 128: 2 waves along M x 4 along N, 64 x 64 each, 3 LDS stages
//             (fp8 weights: the last 1..128 rows of a group).
// fp8 and fp32 256-row tiles give wave wm the 16-row M tiles wm, wm + 4,
// ...: the SIMDs then share a partial tile's valid rows evenly.
// K advances in 128-byte slices: each slice of the TM A rows and the TN B
// rows goes global -> LDS directly (16 bytes per lane per instruction) into
// a ring of NST stages, so the loads run NST - 1 slices ahead of the MFMAs
// and there is one barrier per slice.  With 128-row tiles a stage is 48 KB,
// so three fit and two weight slices (64 KB) per CU stay in flight: the
// medium groups are bound by HBM, and the bytes in flight per CU set the
// bandwidth.  LDS rows are 128 bytes with 16-byte chunk c of row r stored at
// chunk c ^ (r & 7), which keeps the fragment reads of 16 consecutive rows
// free of bank conflicts; the direct loads write chunks in lane order, so
// each lane fetches the global chunk that belongs at its position.  fp8
// scales (one per A row and per B row per slice) go global -> LDS the same
// way: 16 bytes per lane every 4th slice into one of two 4-slice blocks when
// the slice count is a multiple of 4, else 4 bytes per lane per slice.
// Waves whose 64 rows lie beyond the tile's valid rows skip their MFMAs.
// bf16 GEMM1 on 256-row tiles keeps the weight slices three deep and the
// activation slices two deep (160 KB).  For bf16 256-row tiles the direct
// loads go through buffer resources when the offsets fit 32 bits: with the
// global form of the LDS-direct load outstanding, the compiler's wait
// counting waits for every LDS fragment read before each first use, with
// the buffer form it waits for exactly the reads each MFMA needs.

template <int DT, int TM, int TN_ = kTN> struct TileCfg {
  static constexpr int TN = TN_;                              // tile columns
  static constexpr int SL = 128;                              // bytes of K per slice and row
  static constexpr int NST = TM == 256 && TN == 256 ? 2 : 3;  // LDS stages
  static constexpr int CPR = SL / 16;                         // 16-byte chunks per row
  static constexpr int RPI = 1024 / SL;                       // rows one wave instruction fills
  static constexpr int WAVES_M = TM / 64;                     // waves along M (64 rows each)
  static constexpr int WAVES_N = 8 / WAVES_M;                 // waves along N
  static constexpr int WN = TN / WAVES_N;                     // columns per wave
  static constexpr int NTW = WN / 16;                         // 16-column MFMA tiles per wave
  static constexpr int LPA = TM * SL / 1024 / 8;              // A loads per thread per slice
  static constexpr int LPB = TN * SL / 1024 / 8;              // B loads per thread per slice
  static constexpr int NSC = 512;                             // fp8 scale slots per stage: 8 waves x 64
  static constexpr int STAGE = (TM + TN) * SL;                // tile bytes per stage (A then B)
  // fp8 and fp32 256-row tiles: wave wm takes the 16-row M tiles wm, wm + 4,
  // wm + 8, wm + 12 instead of 64 consecutive rows, so that the 4 SIMDs (SIMD
  // s runs waves s and s + 4) share a partial tile's valid rows evenly
  // (tiny_f32, whose groups fill a fraction of a tile: 165 -> 131 us per
  // layer).  bf16 tiles keep consecutive rows: prefill8192_ep8 measured 0.5%
  // slower interleaved.
  static constexpr bool ILV = (DT == MOE_FP8_E4M3 || DT == MOE_F32) && TM == 256;
  // first row of the wave's i-th M tile
  __device__ static __forceinline__ int mrow(int wm, int i) { return ILV ? (i * WAVES_M + wm) * 16 : wm * 64 + i * 16; }
  // the wave's M tiles holding any of the tile's valid rows (they come first in i)
  __device__ static __forceinline__ int mvalid(int wm, int rows) {
    if constexpr (ILV) return min(4, max(0, (((rows + 15) >> 4) - wm + WAVES_M - 1) / WAVES_M));
    else return min(4, max(0, (rows - wm * 64 + 15) >> 4));
  }
  static constexpr int PER_SLICE = LPA + LPB + (DT == MOE_FP8_E4M3 ? 1 : 0);   // loads per thread per slice
  // fp8 scale area: per-slice scales [NST][NSC] floats, or, when the slice
  // count is a multiple of 4, two blocks of [NSC][4 slices] floats
  static constexpr size_t SCB = (size_t)2 * NSC * 16;
  // Epilogue staging of the output tile (bf16 and fp8 layers): TM rows of at
  // most 512 bytes (256 bf16 y columns, or 128 h columns of bf16 or fp32),
  // padded by 16 bytes per row so that the 4 row groups of a wave's writes
  // fall in different LDS banks.
  static constexpr size_t EPI_STRIDE = 512 + 16;
  static constexpr size_t EPI_BYTES = DT == MOE_F32 ? 0 : (size_t)TM * EPI_STRIDE;
  // bf16 256-row tiles: the A rows (gathered activations, mostly fetched
  // from beyond the XCD's L2) in 3 slots and the B rows in 2, so the A loads
  // run two slices ahead of the MFMAs and the B loads one.  160 KB in all.
  // bf16 256-row tiles of GEMM1 keep the weight slices 3 deep and the
  // activation slices 2 deep (the ring below): 5 slots of 32 KB
  static constexpr bool RING_OK = DT == MOE_BF16 && TM == 256;
  static constexpr int SLOT = TM * SL;                        // one operand's slice (TM == TN)
  static constexpr size_t MAIN_BYTES =
      RING_OK ? (size_t)5 * SLOT : (size_t)NST * STAGE + (DT == MOE_FP8_E4M3 ? SCB : 0);
  static constexpr size_t LDS_BYTES = MAIN_BYTES > EPI_BYTES ? MAIN_BYTES : EPI_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  __device__ static __forceinline__ int off(int r, int c) { return r * SL + ((c ^ (r & 7)) << 4); }
};

// Workgroup barrier without the memory fence of __syncthreads(), whose
// release would wait for every outstanding load, including the direct-to-LDS
// loads of later slices that are meant to stay in flight.  The caller first
// waits (vmcnt) for its own loads of the slice about to be read, so after the
// barrier every wave's part of that slice is in LDS; the memory clobber keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// Issue the direct global -> LDS loads of slice kt into stage st.  fp8
// scales (slot 64 * wave + lane): with BLK, a 16-byte load every 4th slice
// fetches 4 slices' scales of the slot's row into block (kt / 4) % 2, so
// each scale row's cache line is touched once per 4 slices (a slice's 512
// scales lie in 512 different rows); else 4 bytes per slice into stage st.
// With SW the weight slices are loaded nontemporally: each is read by about
// one row tile, so it should not displace what other workgroups share.
// Only the wave's first na A-row loads are issued (the others would fetch
// the clamped copies of a partial tile's last row).
template <int DT, int TM, int TN, bool BLK, bool SW>
__device__ __forceinline__ void tile_issue(uint8_t* smem, const uint8_t* const* ga, const uint8_t* const* gb,
                                           const float* gs, int kt, int st, int wave, int na) {
  using C = TileCfg<DT, TM, TN>;
  const size_t off = (size_t)kt * C::SL;
  uint8_t* la = smem + st * C::STAGE + wave * C::LPA * 1024;
  uint8_t* lb = smem + st * C::STAGE + TM * C::SL + wave * C::LPB * 1024;
#pragma unroll
  for (int i = 0; i < C::LPA; ++i)
    if (i < na) __builtin_amdgcn_global_load_lds(ga[i] + off, la + i * 1024, 16, 0, 0);
#pragma unroll
  for (int i = 0; i < C::LPB; ++i) __builtin_amdgcn_global_load_lds(gb[i] + off, lb + i * 1024, 16, 0, SW ? 2 : 0);   // 2: nontemporal
  if constexpr (DT == MOE_FP8_E4M3) {
    uint8_t* sc = smem + C::NST * C::STAGE;
    if constexpr (BLK) {
      if ((kt & 3) == 0) {
        const float* src = gs + kt;
        uint8_t* dst = sc + (((kt >> 2) & 1) * C::NSC + wave * 64) * 16;
        __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
      }
    } else {
      __builtin_amdgcn_global_load_lds(gs + kt, sc + (st * C::NSC + wave * 64) * 4, 4, 0, 0);
    }
  }
}

// One operand's direct loads of a slice (LP per thread) into an LDS slot.
template <bool V> struct BoolC { static constexpr bool value = V; };

template <int LP, bool NT>
__device__ __forceinline__ void issue_rows(uint8_t* slot, const uint8_t* const* g, size_t off, int wave) {
  uint8_t* d = slot + wave * LP * 1024;
#pragma unroll
  for (int i = 0; i < LP; ++i) __builtin_amdgcn_global_load_lds(g[i] + off, d + i * 1024, 16, 0, NT ? 2 : 0);
}

// The same through a buffer resource (32-bit offsets from the resource's
// base; the slice offset in soff).  Same LDS effect; the compiler's wait
// counting then keeps exact LDS-read counts, where with the global form
// pending it waits for every outstanding LDS read before each use.
template <int LP, bool NT>
__device__ __forceinline__ void issue_rows_buf(uint8_t* slot, __amdgpu_buffer_rsrc_t rs, const uint32_t* voff,
                                               int soff, int wave, int n = LP) {
  uint8_t* d = slot + wave * LP * 1024;
#pragma unroll
  for (int i = 0; i < LP; ++i)
    if (i < n)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(d + i * 1024), 16,
                                               (int)voff[i], soff, 0, NT ? 2 : 0);
}

template <int DT, int MODE, bool SHARED, int TM, bool BLK, bool SW, bool BUF>
__global__ __launch_bounds__(512, 1) void ffn_fat_kernel(Args a, int ntn) {
  using F = Frag<DT>;
  using C = TileCfg<DT, TM, tile_cols(DT, MODE, TM, SHARED)>;
  constexpr bool FP8 = DT == MOE_FP8_E4M3;
  constexpr int SL = C::SL, NST = C::NST, RPI = C::RPI, NTW = C::NTW, WN = C::WN;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const float* lds_s = reinterpret_cast<const float*>(smem + NST * C::STAGE);   // fp8: [NST][NSC]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, grp = lane >> 4;
  const int wm = wave / C::WAVES_N, wn = wave % C::WAVES_N;
  const int tile = blockIdx.x / ntn;
  const int nt = blockIdx.x - tile * ntn;
  int g, row0;
  if constexpr (SHARED) {
    // the grid covers exactly the shared expert's tiles of this size: the
    // floor(T / 256) full tiles, or the 128-row tiles of the rest
    g = a.E;
    row0 = TM == 256 ? tile * 256 : (a.T / 256) * 256 + tile * 128;   // 128-row tiles only with mid_rest
  } else {
    if (tile >= a.plan[TM == 256 ? 3 : 4]) return;
    const int32_t* list = a.plan + kPlanHead + 6 * a.G + (TM == 256 ? 0 : 2 * a.fat_cap);
    g = list[2 * tile];
    row0 = list[2 * tile + 1];
  }
  const Group gr = group_of(a, g);
  const int rows = min(TM, gr.m - row0);
  const int K = MODE == 1 ? a.H : a.I;
  const size_t krow = (size_t)K * F::ESZ;
  const int nkt = (int)(krow / SL);
  const int nkb = FP8 ? K / a.qb : 0;

  const uint8_t* asrc = MODE == 1 ? a.a1 : a.a2;
  const uint8_t* wbase;
  const float* wsbase = nullptr;
  if (MODE == 1) {
    wbase = gr.routed ? a.w13 + (size_t)g * 2 * a.I * krow : a.ws13;
    if (FP8) wsbase = gr.routed ? a.w13s + (size_t)g * ((2 * a.I) >> a.wsr_shift) * nkb : a.ws13s;
  } else {
    wbase = gr.routed ? a.w2 + (size_t)g * a.H * krow : a.ws2;
    if (FP8) wsbase = gr.routed ? a.w2s + (size_t)g * (a.H >> a.wsr_shift) * nkb : a.ws2s;
  }
  // Weight row held by LDS B row n; columns past N (a partial last column
  // tile) are clamped to the last valid row and never stored.
  auto b_wrow = [&](int n) -> int {
    if (MODE == 1) {
      const int blk = n >> 4;          // 16-row blocks alternate gate, up
      const int hc = min(nt * (C::TN / 2) + (blk >> 1) * 16 + (n & 15), a.I - 1);
      return ((blk & 1) ? a.I : 0) + hc;
    }
    return min(nt * C::TN + n, a.H - 1);
  };
  // Source row of A row r (clamped: padded rows recompute a valid row, never stored).
  auto a_src = [&](int r) -> int {
    const int rr = r < rows ? r : rows - 1;
    return MODE == 1 ? gemm1_src_row(a, gr, row0 + rr) : gr.slot0 + row0 + rr;
  };
  // This lane's direct-load sources.  Wave instruction i fills LDS rows
  // (wave * LP + i) * RPI + lane / CPR, physical chunk lane % CPR.
  const uint8_t* ga[C::LPA];
  const uint8_t* gb[C::LPB];
#pragma unroll
  for (int i = 0; i < C::LPA; ++i) {
    const int r = (wave * C::LPA + i) * RPI + lane / C::CPR;
    const int lc = (C::off(r, lane % C::CPR) - r * SL) >> 4;   // the swizzle is an involution
    ga[i] = asrc + (size_t)a_src(r) * krow + lc * 16;
  }
#pragma unroll
  for (int i = 0; i < C::LPB; ++i) {
    const int r = (wave * C::LPB + i) * RPI + lane / C::CPR;
    const int lc = (C::off(r, lane % C::CPR) - r * SL) >> 4;
    gb[i] = wbase + (size_t)b_wrow(r) * krow + lc * 16;
  }
  // With BUF (bf16 256-row tiles, when the host finds the activation
  // matrix and one expert's weights below 4 GB) the direct loads go through
  // buffer resources instead: the A base is the activation matrix, the B
  // base this group's weights, with per-lane 32-bit offsets.
  static_assert(!BUF || (DT == MOE_BF16 && TM == 256) || FP8,
                "buffer loads: bf16 256-row tiles and fp8 tiles");
  const __amdgpu_buffer_rsrc_t rsa =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(asrc), 0, (int)0xffffffffu, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wbase), 0, (int)0xffffffffu, 0x00020000);
  uint32_t va[C::LPA], vb[C::LPB];
  if constexpr (BUF) {
#pragma unroll
    for (int i = 0; i < C::LPA; ++i) va[i] = (uint32_t)(ga[i] - asrc);
#pragma unroll
    for (int i = 0; i < C::LPB; ++i) vb[i] = (uint32_t)(gb[i] - wbase);
  }
  // fp8 scales: scale slot s = 64 * wave + lane of each stage holds the
  // slice's scale of A row s (s < TM), of B row s - TM (s < TM + TN), or a
  // copy of B row 0's (the remaining slots, never read).  A wave's slots are
  // all A rows or all B rows, so with BUF its scale resource is one array.
  const float* gs = nullptr;
  const float* sbase = nullptr;
  uint32_t vs = 0;
  if constexpr (FP8) {
    const int sidx = 64 * wave + lane;
    const float* as = MODE == 1 ? a.a1s : a.a2s;
    if (sidx < TM) gs = as + (size_t)a_src(sidx) * nkb;
    else gs = wsbase + (size_t)(b_wrow(sidx < TM + C::TN ? sidx - TM : 0) >> a.wsr_shift) * nkb;
    if constexpr (BUF) {
      const uint64_t sb = reinterpret_cast<uint64_t>(64 * wave < TM ? as : wsbase);
      sbase = reinterpret_cast<const float*>(
          ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(sb >> 32)) << 32) |
          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sb));
      vs = (uint32_t)((gs - sbase) * sizeof(float));
    }
  }

  f32x4 acc[4][NTW];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int mval = C::mvalid(wm, rows);   // this wave's M tiles holding valid rows

  bool full_tile = false;
  if constexpr (!FP8) full_tile = mval == 4;
  constexpr bool RING = C::RING_OK && MODE == 1;
  if constexpr (RING) {
    // GEMM1 on bf16 256-row tiles: the weight (B) slices in 3 LDS slots and
    // the activation (A) slices in 2, 160 KB in all, so the B loads run two
    // slices ahead of the MFMAs and the A loads one.  Slots: B slice kt in
    // slot kt % 3 (at 0, 32, 64 KB), A slice kt in slot kt % 2 (at 96 and
    // 128 KB).  At iteration kt the slots of slice kt - 1 are free after the
    // barrier; A slice kt + 1 is issued first, then B slice kt + 2, so that
    // waiting until only the last LPB loads (B slice kt + 1) are outstanding
    // finds both operands of slice kt landed.  Past the last slice the loads
    // repeat it into a slot nobody reads, which keeps the loop free of
    // branches.  Against two stages of both: prefill8192_ep8 GEMM1 -1%, and
    // -3.5% with the buffer-resource loads.
    auto a_at = [&](int kt) -> uint8_t* { return smem + (3 + (kt & 1)) * C::SLOT; };
    auto b_at = [&](int sd) -> uint8_t* { return smem + sd * C::SLOT; };
    auto issue_a = [&](int kt) {
      const int kk = min(kt, nkt - 1);
      if constexpr (BUF) issue_rows_buf<C::LPA, false>(a_at(kt), rsa, va, kk * SL, wave);
      else issue_rows<C::LPA, false>(a_at(kt), ga, (size_t)kk * SL, wave);
    };
    auto issue_b = [&](int kt, int sd) {
      const int kk = min(kt, nkt - 1);
      if constexpr (BUF) issue_rows_buf<C::LPB, SW>(b_at(sd), rsb, vb, kk * SL, wave);
      else issue_rows<C::LPB, SW>(b_at(sd), gb, (size_t)kk * SL, wave);
    };
    issue_a(0);
    issue_b(0, 0);
    issue_b(1, 1);
    int sd = 0;                                    // kt % 3
    if (full_tile) {
      for (int kt = 0; kt < nkt; ++kt) {
        wait_vmcnt<C::LPB>();                      // this thread's slice kt of both operands has landed
        barrier_no_fence();                        // everyone's has, and slice kt - 1's slots are free
        const uint8_t* la = a_at(kt);
        const uint8_t* lb = b_at(sd);
        const int sd2 = sd == 0 ? 2 : sd - 1;      // (kt + 2) % 3
        i32x4 fa[SL / 64][4], fb[SL / 64][NTW];
#pragma unroll
        for (int fs = 0; fs < SL / 64; ++fs) {
          if (fs == 1) {
            issue_a(kt + 1);
            issue_b(kt + 2, sd2);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            fa[fs][i] = *reinterpret_cast<const i32x4*>(&la[C::off(C::mrow(wm, i) + row, fs * 4 + grp)]);
#pragma unroll
          for (int j = 0; j < NTW; ++j)
            fb[fs][j] = *reinterpret_cast<const i32x4*>(&lb[C::off(wn * WN + j * 16 + row, fs * 4 + grp)]);
        }
#pragma unroll
        for (int fs = 0; fs < SL / 64; ++fs)
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NTW; ++j) F::mma(acc[i][j], fa[fs][i], fb[fs][j]);
        // the same order as the two-stage loop below
        constexpr int R = 4 + NTW;                 // fragment reads per half
        constexpr int L = C::LPA + C::LPB;         // direct loads per slice
        __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
        for (int q = 0; q < L; ++q) {              // 1 load : 2 MFMAs
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
#pragma unroll
        for (int q = 0; q < R; ++q) {              // 1 read : 2 MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8 * NTW - 2 * R - 2 * L, 0);
        sd = sd == 2 ? 0 : sd + 1;
      }
    } else {
      // a group's last, partial tile: the same ring, skipping the M tiles without valid rows
      for (int kt = 0; kt < nkt; ++kt) {
        wait_vmcnt<C::LPB>();
        barrier_no_fence();
        const uint8_t* la = a_at(kt);
        const uint8_t* lb = b_at(sd);
        issue_a(kt + 1);
        issue_b(kt + 2, sd == 0 ? 2 : sd - 1);
        if (mval > 0) {
#pragma unroll
          for (int fs = 0; fs < SL / 64; ++fs) {
            i32x4 fb[NTW];
#pragma unroll
            for (int j = 0; j < NTW; ++j)
              fb[j] = *reinterpret_cast<const i32x4*>(&lb[C::off(wn * WN + j * 16 + row, fs * 4 + grp)]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i < mval) {
                const i32x4 fa = *reinterpret_cast<const i32x4*>(&la[C::off(C::mrow(wm, i) + row, fs * 4 + grp)]);
#pragma unroll
                for (int j = 0; j < NTW; ++j) F::mma(acc[i][j], fa, fb[j]);
              }
          }
        }
        sd = sd == 2 ? 0 : sd + 1;
      }
    }
  } else {
    // A-row loads this wave issues.  fp8 tiles with two stages (the routed
    // 256-row tiles, whose tiles are partial: a group's last 129..255 rows)
    // wait for all of a slice's loads (vmcnt 0), so the loads of 8-row blocks
    // wholly past the valid rows are skipped; their LDS rows feed only C rows
    // that are never stored (serial clustered2048_fp8 256-row GEMM1 -4%).
    // With deeper rings the waits count loads and every load is issued; the
    // bf16 tiles keep a branch-free issue (their GEMM2 measured 4% slower
    // with the test in the full-tile loop).
    const int na = FP8 && NST == 2 ? min(C::LPA, max(0, (rows - wave * C::LPA * RPI + RPI - 1) / RPI)) : C::LPA;
    // slice kt into stage st: A rows, then B rows (and fp8 scales)
    auto tissue = [&](int kt, int st) {
      if constexpr (BUF) {
        issue_rows_buf<C::LPA, false>(smem + st * C::STAGE, rsa, va, kt * SL, wave, na);
        issue_rows_buf<C::LPB, SW>(smem + st * C::STAGE + TM * SL, rsb, vb, kt * SL, wave);
        if constexpr (FP8) {   // the scale loads of tile_issue, from the wave's scale resource
          const __amdgpu_buffer_rsrc_t rss =
              __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sbase), 0, (int)0xffffffffu, 0x00020000);
          uint8_t* sc = smem + C::NST * C::STAGE;
          if constexpr (BLK) {
            if ((kt & 3) == 0)
              __builtin_amdgcn_raw_ptr_buffer_load_lds(
                  rss, (__attribute__((address_space(3))) void*)(sc + (((kt >> 2) & 1) * C::NSC + wave * 64) * 16), 16,
                  (int)vs, kt * 4, 0, 0);
          } else {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rss, (__attribute__((address_space(3))) void*)(sc + (st * C::NSC + wave * 64) * 4), 4, (int)vs, kt * 4,
                0, 0);
          }
        }
      } else {
        tile_issue<DT, TM, C::TN, BLK, SW>(smem, ga, gb, gs, kt, st, wave, na);
      }
    };
#pragma unroll
    for (int p = 0; p < NST - 1; ++p)
      if (p < nkt) tissue(p, p);
    if (full_tile) {
      // Full tiles (all 64 rows of every M tile valid; bf16 and fp32 weights,
      // two stages): one straight-line block per slice, so the scheduling
      // hints below can order the fragment reads, the next slice's direct
      // loads and the MFMAs.  The first half's reads go first; the next slice's
      // loads are issued while they are in flight, spread over the first
      // MFMAs, so a wave never stalls on a full load queue while it has MFMAs
      // ready; the second half's reads are interleaved with the rest of the
      // first half's MFMAs.  The last slice reloads itself into the free stage,
      // which keeps the block free of branches.
      if constexpr (!FP8) {
        static_assert(NST == 2, "the full-tile loop assumes two stages");
        for (int kt = 0; kt < nkt; ++kt) {
          wait_vmcnt<0>();                           // this thread's loads of slice kt have landed
          barrier_no_fence();                        // everyone's have, and the other stage is free
          const uint8_t* la = smem + (kt & 1) * C::STAGE;
          const uint8_t* lb = la + TM * SL;
          i32x4 fa[SL / 64][4], fb[SL / 64][NTW];
#pragma unroll
          for (int fs = 0; fs < SL / 64; ++fs) {
            if (fs == 1) tissue(min(kt + 1, nkt - 1), (kt + 1) & 1);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              fa[fs][i] = *reinterpret_cast<const i32x4*>(&la[C::off(C::mrow(wm, i) + row, fs * 4 + grp)]);
#pragma unroll
            for (int j = 0; j < NTW; ++j)
              fb[fs][j] = *reinterpret_cast<const i32x4*>(&lb[C::off(wn * WN + j * 16 + row, fs * 4 + grp)]);
          }
#pragma unroll
          for (int fs = 0; fs < SL / 64; ++fs)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int j = 0; j < NTW; ++j) F::mma(acc[i][j], fa[fs][i], fb[fs][j]);
          if constexpr (DT == MOE_BF16) {
            constexpr int R = 4 + NTW;                 // fragment reads per half
            constexpr int L = C::LPA + C::LPB;         // direct loads per slice
            __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
            for (int q = 0; q < L; ++q) {              // 1 load : 2 MFMAs
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
#pragma unroll
            for (int q = 0; q < R; ++q) {              // 1 read : 2 MFMAs
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8 * NTW - 2 * R - 2 * L, 0);
          }
        }
      }
    } else {
      for (int kt = 0; kt < nkt; ++kt) {
        const int st = kt % NST;
        // wait until this thread's loads of slice kt have landed; later slices may stay in flight
        if (NST > 2 && kt + 1 < nkt) {
          if (FP8 && BLK) wait_vmcnt_dyn(C::LPA + C::LPB + (((kt + 1) & 3) == 0 ? 1 : 0));
          else wait_vmcnt<C::PER_SLICE>();
        } else {
          wait_vmcnt<0>();
        }
        barrier_no_fence();                          // everyone's slice kt is in LDS; stage (kt-1) % NST is free
        if (kt + NST - 1 < nkt) tissue(kt + NST - 1, (kt + NST - 1) % NST);
        const uint8_t* la = smem + st * C::STAGE;
        const uint8_t* lb = la + TM * SL;
        if constexpr (!FP8) {
          // a group's last, partial tile: skip the M tiles without valid rows
          if (mval > 0) {
#pragma unroll
            for (int fs = 0; fs < SL / 64; ++fs) {
              i32x4 fb[NTW];
#pragma unroll
              for (int j = 0; j < NTW; ++j)
                fb[j] = *reinterpret_cast<const i32x4*>(&lb[C::off(wn * WN + j * 16 + row, fs * 4 + grp)]);
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (i < mval) {
                  const i32x4 fa = *reinterpret_cast<const i32x4*>(&la[C::off(C::mrow(wm, i) + row, fs * 4 + grp)]);
#pragma unroll
                  for (int j = 0; j < NTW; ++j) F::mma(acc[i][j], fa, fb[j]);
                }
            }
          }
        } else {
          // scales of slot s (A row s, then B row s - TM) for slice kt
          constexpr int SS = BLK ? 4 : 1;   // floats between consecutive slots
          const float* sp = BLK ? lds_s + (size_t)((kt >> 2) & 1) * C::NSC * 4 + (kt & 3) : lds_s + st * C::NSC;
          auto scale = [&](int slot) -> float { return sp[slot * SS]; };
          // groups of 4 column tiles keep the B fragments within the register
          // budget; on 128-row tiles a wave whose 4 M tiles all hold valid rows
          // takes a copy without the per-tile guards, which the compiler can
          // software-pipeline (256-row tiles, with 8 column tiles per wave, sit
          // at the register limit and keep only the guarded copy)
#define MOE_FP8_MTILES(GUARD) \
          _Pragma("unroll") \
          for (int jh = 0; jh < NTW / 4; ++jh) { \
            i32x4 fb0[4], fb1[4]; \
            float sb[4]; \
            _Pragma("unroll") \
            for (int jj = 0; jj < 4; ++jj) { \
              const int n = wn * WN + (4 * jh + jj) * 16 + row; \
              fb0[jj] = *reinterpret_cast<const i32x4*>(&lb[C::off(n, grp)]); \
              fb1[jj] = *reinterpret_cast<const i32x4*>(&lb[C::off(n, 4 + grp)]); \
              sb[jj] = scale(TM + n); \
            } \
            _Pragma("unroll") \
            for (int i = 0; i < 4; ++i) { \
              if (GUARD) { \
                const int r = C::mrow(wm, i) + row; \
                const i32x4 fa0 = *reinterpret_cast<const i32x4*>(&la[C::off(r, grp)]); \
                const i32x4 fa1 = *reinterpret_cast<const i32x4*>(&la[C::off(r, 4 + grp)]); \
                float sa[4]; \
                _Pragma("unroll") \
                for (int q = 0; q < 4; ++q) sa[q] = scale(C::mrow(wm, i) + 4 * grp + q); \
                _Pragma("unroll") \
                for (int jj = 0; jj < 4; ++jj) { \
                  const f32x4 p = F::mma128(fa0, fa1, fb0[jj], fb1[jj]); \
                  _Pragma("unroll") \
                  for (int q = 0; q < 4; ++q) \
                    acc[i][4 * jh + jj][q] = fmaf(p[q], sa[q] * sb[jj], acc[i][4 * jh + jj][q]); \
                } \
              } \
            } \
          }
          if (C::NTW == 4 && mval == 4) {
            MOE_FP8_MTILES(true)
          } else {
            MOE_FP8_MTILES(i < mval)
          }
#undef MOE_FP8_MTILES
        }
      }
    }
  }
  wait_vmcnt<0>();   // the loops' last reloads are still in flight

  // ---- epilogue: lane holds rows wm*64 + i*16 + 4*grp + q, columns wn*WN + j*16 + row
  if constexpr (DT != MOE_F32) {
    // Through LDS: each lane writes its values (2-byte bf16, or fp32 h in
    // the fp8 layer) into the row-major output tile, then the workgroup
    // copies whole 16-byte chunks of each row out.  Stored straight from the
    // accumulators, a lane's values are single 2-byte elements 16 columns
    // apart: 64 to 128 scattered store instructions per lane (prefill GEMM2
    // 1742 -> 1699 us staged).
    using OT = typename std::conditional<MODE == 1 && FP8, float, uint16_t>::type;
    constexpr int ES = sizeof(OT);
    constexpr int OC = MODE == 1 ? C::TN / 2 : C::TN;   // output columns of the tile
    constexpr int CPR = OC * ES / 16;                   // 16-byte chunks per row
    constexpr int S = (int)C::EPI_STRIDE;
    static_assert(OC * ES <= 512, "an output row of the tile fits a staging row");
    __syncthreads();                                    // every wave is done with the stages
    uint8_t* lt = smem;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i >= mval) break;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = C::mrow(wm, i) + 4 * grp + q;
        uint8_t* lrow = lt + r * S;
        if (MODE == 1) {
#pragma unroll
          for (int jp = 0; jp < NTW / 2; ++jp) {
            const float v = silu_for<DT>(acc[i][2 * jp][q]) * acc[i][2 * jp + 1][q];
            const int lc = (wn * (NTW / 2) + jp) * 16 + row;
            if constexpr (FP8) reinterpret_cast<float*>(lrow)[lc] = v;
            else reinterpret_cast<uint16_t*>(lrow)[lc] = f32_to_bf16(v);
          }
        } else {
#pragma unroll
          for (int j = 0; j < NTW; ++j) reinterpret_cast<uint16_t*>(lrow)[wn * WN + j * 16 + row] = f32_to_bf16(acc[i][j][q]);
        }
      }
    }
    __syncthreads();
    const int ncols = MODE == 1 ? a.I : a.H;            // row length of h or y (a multiple of 8)
    const int col0 = nt * OC;
    if constexpr (FP8 && MODE == 1 && !SHARED) {
      if (a.tile_quant) {
        // A routed fp8 tile's 128 h columns are one quantisation block of each
        // row (I is a multiple of 128): the tile writes the E4M3 codes and the
        // block's scale, as the quantiser would from the same fp32 values, and
        // h itself never goes to memory.  8 lanes per row, 16 values each.
        static_assert(OC == 128, "one 128-column quantisation block per tile row");
        const int bpr = a.I >> 7;                         // blocks per row of h
        uint8_t* qbase = const_cast<uint8_t*>(a.a2) + (size_t)(gr.slot0 + row0) * a.I + col0;
        float* sbase = const_cast<float*>(a.a2s) + (size_t)(gr.slot0 + row0) * bpr + nt;
        for (int id0 = 0; id0 < rows * 8; id0 += 512) {   // the same trip count for every lane (shuffles)
          const int id = id0 + tid, r = id >> 3, part = id & 7;
          const bool ok = r < rows;
          float v[16];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const f32x4 w = ok ? *reinterpret_cast<const f32x4*>(lt + r * S + part * 64 + c * 16)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < 4; ++q) v[4 * c + q] = w[q];
          }
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
          for (int o = 4; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
          if (ok) {
            const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
            uint32_t w4[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              w4[c] = 0;
#pragma unroll
              for (int q = 0; q < 4; ++q) w4[c] |= f32_to_e4m3(v[4 * c + q] / scale) << (8 * q);
            }
            const i32x4 codes = {(int)w4[0], (int)w4[1], (int)w4[2], (int)w4[3]};
            __builtin_nontemporal_store(codes, reinterpret_cast<i32x4*>(qbase + (size_t)r * a.I + part * 16));
            if (part == 0) sbase[(size_t)r * bpr] = scale;
          }
        }
        return;
      }
    }
    uint8_t* obase = MODE == 1 ? a.h + (size_t)(gr.slot0 + row0) * ncols * ES
                               : (gr.routed ? a.y_sorted : a.y_shared) + (size_t)out_row(a, gr, row0) * ncols * ES;
    for (int id = tid; id < rows * CPR; id += 512) {
      const int r = id / CPR, ch = id - r * CPR;
      const int col = col0 + ch * (16 / ES);
      // Streaming (nontemporal) stores: the tile is written once and the
      // next reader is another launch, so it need not displace the weight
      // and activation panels that neighbouring workgroups share in L2.
      if (col < ncols)
        __builtin_nontemporal_store(
            *reinterpret_cast<const i32x4*>(lt + r * S + ch * 16),
            reinterpret_cast<i32x4*>(obase + ((size_t)r * ncols + col) * ES));
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i >= mval) break;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = C::mrow(wm, i) + 4 * grp + q;
      if (r >= rows) continue;
      if (MODE == 1) {
        const size_t hrow = (size_t)(gr.slot0 + row0 + r) * a.I;
#pragma unroll
        for (int jp = 0; jp < NTW / 2; ++jp) {
          const float gv = acc[i][2 * jp][q], uv = acc[i][2 * jp + 1][q];
          const int col = nt * (C::TN / 2) + (wn * (NTW / 2) + jp) * 16 + row;
          if (col < a.I) store_h<DT>(a.h, hrow + col, silu_for<DT>(gv) * uv);
        }
      } else {
        uint8_t* ybase = gr.routed ? a.y_sorted : a.y_shared;
        const size_t yrow = (size_t)out_row(a, gr, row0 + r) * a.H;
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const int col = nt * C::TN + wn * WN + j * 16 + row;
          if (col < a.H) store_y<DT>(ybase, yrow + col, acc[i][j][q]);
        }
      }
    }
  }
}

template <int DT, int MODE, bool SHARED, int TM, bool BLK, bool SW, bool BUF = false>
hipError_t launch_fat(const char* name, unsigned grid, int ntn, const Args& a, hipStream_t st) {
  using C = TileCfg<DT, TM, tile_cols(DT, MODE, TM, SHARED)>;
  hipError_t e = moe::ensure_dynamic_lds(
      reinterpret_cast<const void*>(&ffn_fat_kernel<DT, MODE, SHARED, TM, BLK, SW, BUF>), (int)C::LDS_BYTES);
  if (e != hipSuccess) return e;
  MOE_LAUNCH(name, (ffn_fat_kernel<DT, MODE, SHARED, TM, BLK, SW, BUF>), dim3(grid), dim3(512), C::LDS_BYTES, st, a,
             ntn);
  return hipGetLastError();
}

}  // namespace

namespace moe {
namespace ffn {

template <int DT>
hipError_t launch_tiled(int mode, bool shared, int tm, bool stream_w, int tiles, const Args& a, hipStream_t st) {
  static const char* const kName[2][2][2] = {                  // [mode - 1][shared][tm == 128]
      {{"ffn_gemm1_tiled", "ffn_gemm1_tiled128"}, {"ffn_gemm1_shared_tiled", "ffn_gemm1_shared_tiled128"}},
      {{"ffn_gemm2_tiled", "ffn_gemm2_tiled128"}, {"ffn_gemm2_shared_tiled", "ffn_gemm2_shared_tiled128"}}};
  const char* name = kName[mode - 1][shared ? 1 : 0][tm == 128 ? 1 : 0];
  // fp8 scale blocks of 4 slices need the slice count K / 128 to be a multiple of 4
  const bool blk = DT == MOE_FP8_E4M3 && (((mode == 1 ? a.H : a.I) / 128) & 3) == 0;
  constexpr bool FP8 = DT == MOE_FP8_E4M3;
  const int ntn = tile_ntn(DT, mode, tm, shared, a.I, a.H);
  const unsigned grid = (unsigned)tiles * (unsigned)ntn;
  // buffer-resource loads (bf16 256-row tiles, fp8 tiles) need 32-bit
  // offsets into the activations (x, or h; fp8: their codes and scales) and
  // into one expert's weights
  const size_t esz = DT == MOE_BF16 ? 2 : 1;
  const size_t act_bytes = mode == 1 ? (size_t)a.T * a.H * esz : (size_t)(a.P + a.T) * a.I * esz;
  const bool buf = (DT == MOE_BF16 ? tm == 256 : FP8) &&
                   act_bytes <= 0xffffffffu && (size_t)2 * a.I * a.H * esz <= 0xffffffffu;
#define MOE_BUFV(M, TMV, S) ((DT == MOE_BF16 && TMV == 256) || FP8)
#define MOE_TLB(M, S, TMV, SWV) \
  (buf ? (FP8 && blk ? launch_fat<DT, M, S, TMV, FP8, SWV, MOE_BUFV(M, TMV, S)>(name, grid, ntn, a, st) \
                     : launch_fat<DT, M, S, TMV, false, SWV, MOE_BUFV(M, TMV, S)>(name, grid, ntn, a, st)) \
       : (FP8 && blk ? launch_fat<DT, M, S, TMV, FP8, SWV>(name, grid, ntn, a, st) \
                     : launch_fat<DT, M, S, TMV, false, SWV>(name, grid, ntn, a, st)))
  // the shared expert's weights are read by every row tile: always cached
#define MOE_TL(M, TMV) \
  (shared ? MOE_TLB(M, true, TMV, false) : stream_w ? MOE_TLB(M, false, TMV, true) : MOE_TLB(M, false, TMV, false))
  if (tm == 256) return mode == 1 ? MOE_TL(1, 256) : MOE_TL(2, 256);
  if constexpr (FP8) return mode == 1 ? MOE_TL(1, 128) : MOE_TL(2, 128);   // 128-row tiles serve fp8 weights only
  return hipErrorInvalidValue;
#undef MOE_TL
#undef MOE_TLB
#undef MOE_BUFV
}

template hipError_t launch_tiled<MOE_F32>(int, bool, int, bool, int, const Args&, hipStream_t);
template hipError_t launch_tiled<MOE_BF16>(int, bool, int, bool, int, const Args&, hipStream_t);
template hipError_t launch_tiled<MOE_FP8_E4M3>(int, bool, int, bool, int, const Args&, hipStream_t);

}  // namespace ffn
}  // namespace moe
