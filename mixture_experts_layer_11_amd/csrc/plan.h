// The expert FFN's work lists, built by one workgroup from the per-group row
// counts: three streaming classes by row count (1-8, 9-16, 17-32 rows) and
// the 256-row and 128-row tile lists, each by a prefix sum over the groups.
// Used by the FFN's own plan kernel and by the one-workgroup dispatch, which
// holds the counts already.
#pragma once

#include "ffn.h"

namespace moe {
namespace ffn {

// LDS ints build_plan needs from its caller.
constexpr int kPlanLds = 5 * 8 + 2 * 8 + 3 * 512;

// Thread g (any block of at least 512 threads; all threads must call it)
// owns group g with m rows (0 for g >= G).  wt holds kPlanLds ints of LDS.
// Skinny class: 0 for 1..8 rows, 1 for 9..16, 2 for 17..32; larger groups
// take floor(m / 256) full tiles, and their last m mod 256 rows one more
// 256-row tile, or with mid_rest one 128-row tile if they are at most 128
// (one 256-row tile above that, which reads the weights once).  The shared
// expert (g == E) has launches of its own, except in halves mode (T <= 16):
// there every group, the shared expert included, enters the <= 8-row list
// as one or two 8-row halves, so the other lists stay empty; and with
// shared_tiled, where its tiles join the routed tile lists like a group of
// T rows.  The five
// per-group counts are prefix-summed over groups 0..g in each wave with
// shuffles, then across the 8 waves through wt (one barrier).  The two tile
// lists run in order of decreasing group size (equal sizes by group), so a
// launch ends with the smallest groups' tiles and its last workgroups are
// short ones; a group's row tiles stay consecutive.
__device__ inline void build_plan(const PlanArgs& a, int m, int* wt) {
  const int g = threadIdx.x, lane = g & 63, wave = g >> 6;
  const bool act = g < 512;
  const bool shared = g == a.E;
  const bool listed = m > 0 && m <= kSkinnyRows && (!shared || a.halves);
  const int cls = listed ? (a.halves || m <= 8 ? 0 : m <= 16 ? 1 : 2) : -1;
  const int nent = cls < 0 ? 0 : (a.halves ? (m + 7) / 8 : 1);   // list entries of this group
  const bool tiled = m > kSkinnyRows && (!shared || a.shared_tiled);
  const int rest = m % kTileRows;
  const bool rest_fat = a.mid_rest && rest > kMidRows;   // one partial 256-row tile reads the weights once
  const int tiles = tiled ? (a.mid_rest ? m / kTileRows + (rest_fat ? 1 : 0) : (m + kTileRows - 1) / kTileRows) : 0;
  const int mids = tiled && a.mid_rest && !rest_fat ? (rest + kMidRows - 1) / kMidRows : 0;
  // [0..2] skinny list entries by class, [3] 256-row tiles, [4] 128-row tiles
  int v[5] = {cls == 0 ? nent : 0, cls == 1 ? nent : 0, cls == 2 ? nent : 0, tiles, mids};
#pragma unroll
  for (int c = 0; c < 5; ++c) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int u = __shfl_up(v[c], d, 64);
      if (lane >= d) v[c] += u;
    }
  }
  if (act && lane == 63) {
#pragma unroll
    for (int c = 0; c < 5; ++c) wt[c * 8 + wave] = v[c];
  }
  __syncthreads();
  int32_t* plan = a.plan;
  if (act) {   // every thread of the block reaches the barriers below
    for (int w = 0; w < wave; ++w) {
#pragma unroll
      for (int c = 0; c < 5; ++c) v[c] += wt[c * 8 + w];
    }
    // v[c] now sums groups 0..g
    if (g == 511) {
#pragma unroll
      for (int c = 0; c < 5; ++c) plan[c] = v[c];
    }
    const int send = cls == 0 ? v[0] : cls == 1 ? v[1] : v[2];   // end of this group's entries in its list
    for (int h = 0; h < nent; ++h) plan[kPlanHead + cls * 2 * a.G + send - nent + h] = g | (h << 16);
  }

  // Tile lists by decreasing group size: rank r of each tiled group, its
  // tile counts at position r, a prefix sum over positions, and back.
  int* wp = wt + 5 * 8;        // [2][8] cross-wave sums
  int* ms = wp + 2 * 8;        // [512] rows of tiled groups (-1: not tiled)
  int* ct = ms + 512;          // [512] 256-row tiles at position r, then their start
  int* cm = ct + 512;          // [512] 128-row tiles at position r, then their start
  const bool ranked = act && (tiles > 0 || mids > 0);
  if (act) {
    ms[g] = ranked ? m : -1;
    ct[g] = 0;
    cm[g] = 0;
  }
  __syncthreads();
  int r = 0;
  if (ranked) {
    for (int h = 0; h < a.G; ++h) {
      const int mh = ms[h];
      r += mh > m || (mh == m && h < g);
    }
    ct[r] = tiles;
    cm[r] = mids;
  }
  __syncthreads();
  int u[2] = {act ? ct[g] : 0, act ? cm[g] : 0};   // thread g now stands for position g
  const int own[2] = {u[0], u[1]};
#pragma unroll
  for (int c = 0; c < 2; ++c) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int w = __shfl_up(u[c], d, 64);
      if (lane >= d) u[c] += w;
    }
  }
  if (act && lane == 63) {
    wp[wave] = u[0];
    wp[8 + wave] = u[1];
  }
  __syncthreads();
  if (act) {
    for (int w = 0; w < wave; ++w) {
      u[0] += wp[w];
      u[1] += wp[8 + w];
    }
    ct[g] = u[0] - own[0];     // start of position g's tiles (position g read its own count above)
    cm[g] = u[1] - own[1];
  }
  __syncthreads();
  if (!ranked) return;
  int32_t* fat = plan + kPlanHead + 6 * a.G;
  const int t0 = ct[r];
  for (int i = 0; i < tiles; ++i) {
    fat[2 * (t0 + i)] = g;
    fat[2 * (t0 + i) + 1] = i * kTileRows;
  }
  int32_t* mid = fat + 2 * a.fat_cap;
  const int m0 = cm[r];
  for (int i = 0; i < mids; ++i) {
    mid[2 * (m0 + i)] = g;
    mid[2 * (m0 + i) + 1] = (m / kTileRows) * kTileRows + i * kMidRows;
  }
}

}  // namespace ffn
}  // namespace moe
