// The expert FFN's work lists, built by one workgroup from the per-group row
// counts: three streaming classes by row count (1-8, 9-16, 17-32 rows) and
// the 256-row and 128-row tile lists, each by an LDS prefix sum over the
// groups.  Used by the FFN's own plan kernel and by the one-workgroup
// dispatch, which holds the counts already.
#pragma once

#include "ffn.h"

namespace moe {
namespace ffn {

// Thread g (any block of at least 512 threads; all threads must call it)
// owns group g with m rows (0 for g >= G).  sk holds 3 x 512 ints, ft and mt
// 512 each, all in LDS.  Skinny class: 0 for 1..8 rows, 1 for 9..16, 2 for
// 17..32; larger groups take floor(m / 256) full tiles, and their last
// m mod 256 rows one more 256-row tile, or with mid_rest one 128-row tile if
// they are at most 128 (one 256-row tile above that, which reads the weights
// once).  The shared expert (g == E) has launches of its own, except in
// halves mode (T <= 16): there every group, the shared expert included,
// enters the <= 8-row list as one or two 8-row halves, so the other lists
// stay empty.
__device__ inline void build_plan(const PlanArgs& a, int m, int* sk, int* ft, int* mt) {
  const int g = threadIdx.x;
  const bool act = g < 512;
  const bool shared = g == a.E;
  const bool listed = m > 0 && m <= kSkinnyRows && (!shared || a.halves);
  const int cls = listed ? (a.halves || m <= 8 ? 0 : m <= 16 ? 1 : 2) : -1;
  const int nent = cls < 0 ? 0 : (a.halves ? (m + 7) / 8 : 1);   // list entries of this group
  const bool tiled = m > kSkinnyRows && !shared;
  const int rest = m % kTileRows;
  const bool rest_fat = a.mid_rest && rest > kMidRows;   // one partial 256-row tile reads the weights once
  const int tiles = tiled ? (a.mid_rest ? m / kTileRows + (rest_fat ? 1 : 0) : (m + kTileRows - 1) / kTileRows) : 0;
  const int mids = tiled && a.mid_rest && !rest_fat ? (rest + kMidRows - 1) / kMidRows : 0;
  if (act) {
#pragma unroll
    for (int c = 0; c < 3; ++c) sk[c * 512 + g] = cls == c ? nent : 0;
    ft[g] = tiles;
    mt[g] = mids;
  }
  __syncthreads();
  for (int d = 1; d < 512; d <<= 1) {
    int v[3] = {0, 0, 0}, v2 = 0, v3 = 0;
    if (act && g >= d) {
#pragma unroll
      for (int c = 0; c < 3; ++c) v[c] = sk[c * 512 + g - d];
      v2 = ft[g - d];
      v3 = mt[g - d];
    }
    __syncthreads();
    if (act) {
#pragma unroll
      for (int c = 0; c < 3; ++c) sk[c * 512 + g] += v[c];
      ft[g] += v2;
      mt[g] += v3;
    }
    __syncthreads();
  }
  if (!act) return;
  int32_t* plan = a.plan;
  if (g == 511) {
#pragma unroll
    for (int c = 0; c < 3; ++c) plan[c] = sk[c * 512 + 511];
    plan[3] = ft[511];
    plan[4] = mt[511];
  }
  for (int h = 0; h < nent; ++h) plan[kPlanHead + cls * 2 * a.G + sk[cls * 512 + g] - nent + h] = g | (h << 16);
  int32_t* fat = plan + kPlanHead + 6 * a.G;
  const int t0 = ft[g] - tiles;
  for (int i = 0; i < tiles; ++i) {
    fat[2 * (t0 + i)] = g;
    fat[2 * (t0 + i) + 1] = i * kTileRows;
  }
  int32_t* mid = fat + 2 * a.fat_cap;
  const int m0 = mt[g] - mids;
  for (int i = 0; i < mids; ++i) {
    mid[2 * (m0 + i)] = g;
    mid[2 * (m0 + i) + 1] = (m / kTileRows) * kTileRows + i * kMidRows;
  }
}

}  // namespace ffn
}  // namespace moe
