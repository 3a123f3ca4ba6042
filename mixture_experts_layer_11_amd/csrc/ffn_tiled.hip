// Tiled grouped GEMM: expert groups of more than 32 rows (prefill), and the
// shared expert beyond 32 tokens, on MFMA tiles with LDS-staged operands.
//
// Perplexity's "Lower latency and higher throughput with multi-node DeepSeek
// deployment" (sections "GroupGEMM" and "Future work") finds the grouped
// GEMM compute-bound once the rows per expert are many.

#include "ffn.h"

namespace {

using namespace moe::ffn;

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

template <int DT, int MODE, bool SHARED>
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
  if constexpr (SHARED) {          // the grid covers exactly ceil(T / kTM) row tiles of the shared expert
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

template <int DT, int MODE, bool SHARED>
hipError_t launch_fat(const char* name, unsigned grid, int ntn, const Args& a, hipStream_t st) {
  constexpr bool FP8 = DT == MOE_FP8_E4M3;
  using C = TileCfg<DT>;
  const size_t smem = (size_t)C::NST * C::STAGE + (FP8 ? C::NST * (kTM + kTN) * sizeof(float) : 0);
  static bool attr_set = false;   // raise the dynamic-LDS limit once per process
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&ffn_fat_kernel<DT, MODE, SHARED>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  MOE_LAUNCH(name, (ffn_fat_kernel<DT, MODE, SHARED>), dim3(grid), dim3(512), smem, st, a, ntn);
  return hipGetLastError();
}

}  // namespace

namespace moe {
namespace ffn {

template <int DT>
hipError_t launch_tiled(int mode, bool shared, unsigned grid, int ntn, const Args& a, hipStream_t st) {
  if (mode == 1)
    return shared ? launch_fat<DT, 1, true>("ffn_gemm1_shared_tiled", grid, ntn, a, st)
                  : launch_fat<DT, 1, false>("ffn_gemm1_tiled", grid, ntn, a, st);
  return shared ? launch_fat<DT, 2, true>("ffn_gemm2_shared_tiled", grid, ntn, a, st)
                : launch_fat<DT, 2, false>("ffn_gemm2_tiled", grid, ntn, a, st);
}

template hipError_t launch_tiled<MOE_F32>(int, bool, unsigned, int, const Args&, hipStream_t);
template hipError_t launch_tiled<MOE_BF16>(int, bool, unsigned, int, const Args&, hipStream_t);
template hipError_t launch_tiled<MOE_FP8_E4M3>(int, bool, unsigned, int, const Args&, hipStream_t);

}  // namespace ffn
}  // namespace moe
