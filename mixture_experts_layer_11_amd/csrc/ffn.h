// Expert FFN internals shared by the planner and launcher (ffn.hip), the
// streaming "skinny" kernels (ffn_skinny.hip) and the tiled kernels
// (ffn_tiled.hip): the kernel argument block, group bookkeeping, output
// stores, the regime and tile constants and the per-file launchers.
#pragma once

#include "moe_common.h"
#include "moe_launch.h"

namespace moe {
namespace ffn {

constexpr int kSkinnyRows = 32;  // groups with <= this many rows take the skinny path
constexpr int kTileRows = 256;   // rows per full tile of the tiled grouped GEMM
constexpr int kMidRows = 128;    // rows per tile for the rest of a group (m mod 256 rows), fp8 weights
// The shared expert joins the routed tile lists when it is tiled, has no
// fp8 quantisation between its GEMMs, and its GEMM1 alone has at least this
// many 256 x 256 tiles (MI355X's CU count: it fills the device and is not
// overlapped with the routed work, e.g. the 8192-token prefill share): one
// launch per GEMM then covers both, without a tail between them.
constexpr int kSharedInListTiles = 256;
constexpr int kPlanHead = 5;     // plan: [0..2] skinny list sizes (<=8, <=16, <=32 rows), [3] 256-row tiles,
                                 // [4] 128-row tiles

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
  int wsr_shift;                // fp8 weight scales: row r uses scale row r >> wsr_shift (0: 1 x 128, 7: 128 x 128)
  uint8_t* h;                   // GEMM1 out [P+T, I]
  const uint8_t* a2;            // GEMM2 A rows: h or fp8 codes of h, [P+T, I]
  const float* a2s;             // fp8: h scales [P+T, I/qb]
  uint8_t* y_sorted;            // act dtype (fp32 when DT is fp32, else bf16)
  uint8_t* y_shared;
  const int32_t* plan;          // see ffn_plan_kernel: list sizes, 3 skinny lists of 2G, tile (group,row0) pairs
  int G;
  int halves;                   // T <= 16: every group in the <= 8-row list, in 8-row halves (shared expert too)
  int fat_cap;                  // capacity of the plan's 256-row tile list (the 128-row list follows it)
  int mid_rest;                 // 1: a group's last m mod 256 rows take 128-row tiles; 0: one more 256-row tile
  int shared_tiled;             // 1: the shared expert (group E) is in the routed tile lists, no launches of its own
  int first_mode;               // host side: 1 runs GEMM1 then GEMM2; 2 runs GEMM2 alone on the h in place
  int tile_quant;               // fp8: routed GEMM1 tiles write h's codes and scales instead of h
};

struct Group {
  int m;         // rows
  int slot0;     // first row in the [P+T] row space of h (routed: offsets[g]; shared: P + first token)
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

// A skinny list entry: group g (low 16 bits) and, in halves mode, which
// 8-row half of it (bit 16): the half's rows start 8 rows further in h.
__device__ __forceinline__ Group group_of_entry(const Args& a, int ent, int* g) {
  *g = ent & 0xFFFF;
  Group r = group_of(a, *g);
  if (a.halves) {                 // entry = rows [8 * half, 8 * half + 8) of the group
    const int half = ent >> 16;
    r.slot0 += 8 * half;
    r.m = min(8, r.m - 8 * half);
  }
  return r;
}

// Token (row of x) feeding row r of group g in GEMM1 (the shared expert's
// rows are the tokens, from P on in h's row space).
__device__ __forceinline__ int gemm1_src_row(const Args& a, const Group& gr, int r) {
  return gr.routed ? a.sorted_pair[gr.slot0 + r] / a.k : gr.slot0 - a.P + r;
}

// Row of y_sorted (routed) or y_shared (shared) for row r of a group.
__device__ __forceinline__ int out_row(const Args& a, const Group& gr, int r) {
  return gr.routed ? gr.slot0 + r : gr.slot0 - a.P + r;
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

// s_waitcnt that waits for vmcnt <= n only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// vmcnt <= n for a wave-uniform n known only at run time (0 <= n < 48).
__device__ __forceinline__ void wait_vmcnt_dyn(int n) {
#define MOE_WC(K) \
  case K:         \
    wait_vmcnt<K>(); \
    break;
#define MOE_WC8(K) MOE_WC(K) MOE_WC(K + 1) MOE_WC(K + 2) MOE_WC(K + 3) MOE_WC(K + 4) MOE_WC(K + 5) MOE_WC(K + 6) MOE_WC(K + 7)
  switch (n) {
    MOE_WC8(0) MOE_WC8(8) MOE_WC8(16) MOE_WC8(24) MOE_WC8(32) MOE_WC8(40)
    default: wait_vmcnt<0>();
  }
#undef MOE_WC8
#undef MOE_WC
}

// s_waitcnt lgkmcnt(0) only: this wave's LDS reads have completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// 8-row weight tiles per routed skinny item (GEMM1: gate/up halves, so a
// multiple of 4).  bf16 GEMM1 takes half-width items: each workgroup's work
// then lasts half as long, which halves the launch's draining tail, where
// fewer and fewer CUs keep loads in flight (decode16 GEMM1 748 -> 730 us);
// elsewhere the wider items measured faster.
__host__ __device__ constexpr int sk_nt(int dt, int mode) { return dt == MOE_BF16 && mode == 1 ? 4 : 8; }
constexpr int kShNT = 2;   // 8-row weight tiles per item of the skinny shared expert
constexpr int kShKS = 4;   // waves splitting K in the skinny shared expert's workgroups
constexpr int kTM = 256;   // tiled GEMM: tile rows (tokens)
constexpr int kTN = 256;   // tiled GEMM: tile columns (weight rows; GEMM1: 128 gate + 128 up)

// Tile columns of the tiled GEMM with TM-row tiles: kTN, except for the fp8
// shared expert's 256-row GEMM1 tiles, which take 128 columns (64 gate + 64
// up): three LDS stages and 64 accumulators per wave then fit, which suits
// its full, compute-bound tiles over K = H (clustered2048_fp8, alone: 173 ->
// 107 us).  Its GEMM2 (K = I, 16 slices) measured 60 -> 65 us that way and
// keeps kTN.  The routed fp8 256-row tiles are partial (129..255 rows left
// of a group) and bound by their loads, which the narrower tiles' twice
// re-read activation rows make slower (GEMM1 439 -> 461 us): they keep kTN.
__host__ __device__ constexpr int tile_cols(int dt, int mode, int tm, bool shared) {
  return dt == MOE_FP8_E4M3 && mode == 1 && tm == 256 && shared ? 128 : kTN;
}
// Column tiles per row tile: GEMM1 covers I h-columns (half of a tile's
// weight rows are gate rows), GEMM2 the H output columns.
inline int tile_ntn(int dt, int mode, int tm, bool shared, int I, int H) {
  const int tn = tile_cols(dt, mode, tm, shared);
  return mode == 1 ? (I + tn / 2 - 1) / (tn / 2) : (H + tn - 1) / tn;
}

// Launchers (explicitly instantiated for MOE_F32, MOE_BF16, MOE_FP8_E4M3).
// mode 1 = gate/up GEMM with SwiGLU, mode 2 = down GEMM.
// The routed skinny classes (1..8, 9..16, 17..32 rows) in one launch of `grid` workgroups.
template <int DT>
hipError_t launch_skinny(int mode, unsigned grid, const Args& a, hipStream_t st);
// The shared expert when T <= kSkinnyRows.
template <int DT>
hipError_t launch_shared_skinny(int mode, int T, const Args& a, hipStream_t st);
// Tiled grouped GEMM with tm-row tiles (256 or 128): the plan's list of that
// size (shared = false) or the shared expert's tiles of that size (shared =
// true: floor(T / 256) full tiles, or ceil((T mod 256) / 128) tiles for the
// rest), for `tiles` row tiles of tile_ntn column tiles each (the routed
// lists' row tiles beyond the plan's count exit at once).  stream_w (routed
// tiles only) loads the weight slices nontemporally, for when each group's
// weights are read by about one row tile.
template <int DT>
hipError_t launch_tiled(int mode, bool shared, int tm, bool stream_w, int tiles, const Args& a, hipStream_t st);

}  // namespace ffn
}  // namespace moe
