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
//                 regimes: "skinny" groups with 1..kSkinnyRows rows (in three
//                 classes by row count) and "fat" groups, cut into
//                 kTileRows-row tiles (fp8: the last 1..128 rows of a group
//                 into one kMidRows-row tile).
//   skinny GEMM   (ffn_skinny.hip) one wave takes an item of 64 weight rows
//                 and streams its 128-byte K windows global -> LDS through a
//                 ring of its own (each weight byte is read once) against
//                 the group's <= 32 rows.  Bandwidth-bound decode regime.
//   tiled GEMM    (ffn_tiled.hip) 256 x 256 (or 128 x 256) output tiles per
//                 workgroup, K staged through LDS in 128-byte slices loaded
//                 global -> LDS directly, 8 waves with 16x16 MFMAs.
//                 Compute-bound prefill regime.
//
// GEMM1 (mode 1) produces h = SiLU(A W1^T) * (A W3^T): every output tile holds
// matching gate and up columns (16-column blocks interleaved gate, up, gate,
// up), so SwiGLU is applied in registers.  GEMM2 (mode 2) is the down
// projection into y_sorted (routed) or y_shared.
//
// FP8 E4M3 weights carry one fp32 scale per row (or per 128 rows) per 128
// K-values and the activations one scale per row per 128: each 128-wide K
// block is one 16x16x128 MFMA with unit block exponents, promoted to fp32
// with scale_a[row] * scale_w[col] and accumulated on the vector ALU.

#include "ffn.h"
#include "plan.h"

namespace {

using namespace moe::ffn;

// ------------------------------------------------------------------ plan

__global__ __launch_bounds__(512) void ffn_plan_kernel(Args a) {
  __shared__ int wt[moe::ffn::kPlanLds];
  const int g = threadIdx.x;
  int m = 0;
  if (g < a.G) m = g < a.E ? a.offsets[g + 1] - a.offsets[g] : a.T;
  build_plan(moe::PlanArgs{const_cast<int32_t*>(a.plan), a.G, a.E, a.T, a.fat_cap, a.halves, a.mid_rest,
                           a.shared_tiled},
             m, wt);
}

// fp8 with tile_quant: the routed tiles quantise their rows of h in GEMM1's
// epilogue, so only the streaming groups' rows (routed groups of 1 to
// kSkinnyRows rows) are quantised here, from the fp32 h the streaming GEMM1
// wrote, with the quantiser's arithmetic.  Workgroup (g, y) takes routed
// group g (exiting unless it streams) and the y-th of kQuantSplit equal
// shares of its 128-value blocks; 16 lanes per block, 8 values each, and
// each lane loads the values of its kQuantUnroll blocks before reducing any,
// so that a group of up to 32 rows takes one or two rounds of loads.
constexpr int kQuantSplit = 4, kQuantUnroll = 4;

__global__ __launch_bounds__(256) void quant_skinny_rows_kernel(Args a) {
  const int g = blockIdx.x;
  const int r0 = a.offsets[g], m = a.offsets[g + 1] - r0, bpr = a.I >> 7;
  if (m == 0 || m > kSkinnyRows) return;
  const int nblk = m * bpr;
  const int b_end = (int)((long long)nblk * (blockIdx.y + 1) / kQuantSplit);
  const float* h = reinterpret_cast<const float*>(a.h) + (size_t)r0 * a.I;
  uint8_t* hq = const_cast<uint8_t*>(a.a2) + (size_t)r0 * a.I;
  float* hs = const_cast<float*>(a.a2s) + (size_t)r0 * bpr;
  const int l = threadIdx.x & 15;
  // the same trip count for every lane (shuffles)
  for (int b0 = (int)((long long)nblk * blockIdx.y / kQuantSplit); b0 < b_end; b0 += 16 * kQuantUnroll) {
    float v[kQuantUnroll][8];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const int b = b0 + 16 * u + (threadIdx.x >> 4);   // block b of the group's rows
      if (b < b_end) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(h + (size_t)b * 128 + l * 8);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(h + (size_t)b * 128 + l * 8 + 4);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[u][q] = lo[q];
          v[u][4 + q] = hi[q];
        }
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) v[u][q] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const int b = b0 + 16 * u + (threadIdx.x >> 4);
      float amax = 0.f;
#pragma unroll
      for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[u][q]));
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      if (b >= b_end) continue;
      const float scale = amax == 0.f ? 1.0f : amax / 448.0f;
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lo |= f32_to_e4m3(v[u][q] / scale) << (8 * q);
        hi |= f32_to_e4m3(v[u][4 + q] / scale) << (8 * q);
      }
      *reinterpret_cast<uint2*>(hq + (size_t)b * 128 + l * 8) = make_uint2(lo, hi);
      if (l == 0) hs[b] = scale;
    }
  }
}

// The shared expert: its own launches, on the stream it is given.
template <int DT>
hipError_t run_shared(const moe_cfg& c, const Args& a, hipStream_t st) {
  const int P = a.P;
  hipError_t e;
  for (int mode = a.first_mode; mode <= 2; ++mode) {
    if (mode == 2 && DT == MOE_FP8_E4M3 && a.first_mode == 1) {   // its rows [P, P + T) of h
      e = moe::launch_quant_fp8(c.T, c.I, a.qb, a.h + (size_t)P * c.I * 4, MOE_F32,
                                const_cast<uint8_t*>(a.a2) + (size_t)P * c.I,
                                const_cast<float*>(a.a2s) + (size_t)P * (c.I / a.qb), st);
      if (e != hipSuccess) return e;
    }
    if (c.T <= kSkinnyRows) {
      e = launch_shared_skinny<DT>(mode, c.T, a, st);
    } else {
      const int full = a.mid_rest ? c.T / kTileRows : moe::ceil_div(c.T, kTileRows);
      const int rest = a.mid_rest ? moe::ceil_div(c.T % kTileRows, kMidRows) : 0;
      e = hipSuccess;
      if (full > 0) e = launch_tiled<DT>(mode, true, kTileRows, false, full, a, st);
      if (e == hipSuccess && rest > 0) e = launch_tiled<DT>(mode, true, kMidRows, false, rest, a, st);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// The routed experts, on the stream it is given: plan, then per projection
// the three skinny classes and the tiled groups.  Grids are sized on the
// host from upper bounds; workgroups beyond the device-side lists exit.
// run_routed calls hook(2 * mode - 2) at the start of each GEMM's stage (mode
// 1, 2; for fp8 before the quantisation of h) and hook(2 * mode - 1) after
// its streaming launch; run_ffn forks the shared expert there.
struct NoHook {
  hipError_t operator()(int) const { return hipSuccess; }
};

template <int DT, typename Hook = NoHook>
hipError_t run_routed(const moe_cfg& c, const Args& a, hipStream_t st, bool planned, bool fork,
                      const Hook& hook = Hook()) {
  hipError_t e;
  if (!planned) {   // else the dispatch built the plan already
    MOE_LAUNCH("ffn_plan", ffn_plan_kernel, dim3(1), dim3(512), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int P = a.P;
  // Upper bounds of the tile lists: a token picks k distinct experts, so a
  // routed group has at most T rows and none is tiled when T <= kSkinnyRows.
  // Otherwise at most P / 256 full tiles plus one partial tile per tiled
  // group (256 rows, or with mid_rest 128 rows), of which there are at most
  // min(E, P / (kSkinnyRows + 1)).
  int tiled_groups = c.T > kSkinnyRows ? (P / (kSkinnyRows + 1) < c.E ? P / (kSkinnyRows + 1) : c.E) : 0;
  // With mid_rest every 256-row tile, full or partial, holds more than 128 of
  // the P rows, so there are also at most P / 129 of them (clustered2048_fp8:
  // 127 instead of 320 tiles in the grid, the rest exiting at once).
  int max_fat = tiled_groups > 0 ? P / kTileRows + tiled_groups : 0;
  if (a.mid_rest && P / (kMidRows + 1) < max_fat) max_fat = P / (kMidRows + 1);
  if (a.shared_tiled) {   // the shared expert's ceil(T / 256) tiles join the list (never with mid_rest)
    max_fat += moe::ceil_div(c.T, kTileRows);
    tiled_groups += 1;
  }
  const int max_mid = a.mid_rest ? tiled_groups : 0;
  // halves mode: the shared expert's rows [P, P + T) of h are the routed lists' too
  const int qrows = P + (a.halves && a.has_shared ? c.T : 0);
  for (int mode = a.first_mode; mode <= 2; ++mode) {
    if ((e = hook(2 * mode - 2)) != hipSuccess) return e;
    if (mode == 2 && DT == MOE_FP8_E4M3 && a.first_mode == 1) {
      if (a.tile_quant) {   // the tiles quantised theirs; the streaming groups' rows remain
        MOE_LAUNCH("quant_fp8_skinny_rows", quant_skinny_rows_kernel, dim3(c.E, kQuantSplit), dim3(256), 0, st, a);
        e = hipGetLastError();
      } else {
        e = moe::launch_quant_fp8(qrows, c.I, a.qb, a.h, MOE_F32, const_cast<uint8_t*>(a.a2),
                                  const_cast<float*>(a.a2s), st);
      }
      if (e != hipSuccess) return e;
    }
    const int N = mode == 1 ? c.I : c.H;
    const long long items = N / ((mode == 1 ? 4 : 8) * sk_nt(DT, mode));   // skinny items per group
    long long bands = 0;   // workgroups per XCD over the three class bands (the kernel's order)
    for (int cls = 0; cls < 3; ++cls) {
      // a group of class cls has at least 1, 9 or 17 rows, and no group has
      // more than T rows (a token picks k distinct experts)
      const int min_rows = cls == 0 ? 1 : (4 << cls) + 1;
      int groups = P / min_rows < c.E ? P / min_rows : c.E;
      if (a.halves) {            // every half has at least one row; two halves of the shared expert
        if (cls > 0) continue;
        groups = (P < 2 * c.E ? P : 2 * c.E) + (a.has_shared ? 2 : 0);
      }
      if (groups == 0 || min_rows > c.T) continue;
      bands += moe::ceil_div(moe::ceil_div(groups * items, 4LL), 8LL);   // 4 items per workgroup
    }
    // When both regimes are expected (a mean of 17..1023 rows per routed
    // expert), the tiled launches go on a second side stream, forked before
    // the streaming launch and joined after it, so the two share the device
    // instead of running one after the other (clustered2048_fp8: 2.70 ->
    // 2.62 ms).  Outside that range one regime is empty or nearly so and the
    // fork and join only add latency (prefill8192_ep8: +40 us).
    const int mean_rows = P / c.E;
    const bool both = fork && bands > 0 && (max_fat > 0 || max_mid > 0) && mean_rows > kSkinnyRows / 2 &&
                      mean_rows < 4 * kTileRows;
    // With a mean of at most one 256-row tile per routed expert, most groups'
    // weights are read by one row tile, and nontemporal loads keep them from
    // displacing the activation rows that the column tiles share
    // (clustered2048_fp8: 2.54 -> 2.50 ms).  With more row tiles per group
    // the weights must stay cached (prefill8192_ep8: 5.72 -> 6.37 ms).
    const bool stream_w = mean_rows <= kTileRows;
    hipStream_t tst = st;
    moe::SideStream ts{};
    if (both) {
      if ((e = moe::side_stream(&ts, 1)) != hipSuccess) return e;
      if ((e = hipEventRecord(ts.fork, st)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(ts.stream, ts.fork, 0)) != hipSuccess) return e;
      tst = ts.stream;
    }
    if (both) {   // tiles first, so their workgroups are queued before the streaming ones
      if (max_fat > 0 && (e = launch_tiled<DT>(mode, false, kTileRows, stream_w, max_fat, a, tst)) != hipSuccess)
        return e;
      if (max_mid > 0 && (e = launch_tiled<DT>(mode, false, kMidRows, stream_w, max_mid, a, tst)) != hipSuccess)
        return e;
    }
    if (bands > 0 && (e = launch_skinny<DT>(mode, (unsigned)(8 * bands), a, st)) != hipSuccess) return e;
    if ((e = hook(2 * mode - 1)) != hipSuccess) return e;
    if (!both) {
      if (max_fat > 0 && (e = launch_tiled<DT>(mode, false, kTileRows, stream_w, max_fat, a, st)) != hipSuccess)
        return e;
      if (max_mid > 0 && (e = launch_tiled<DT>(mode, false, kMidRows, stream_w, max_mid, a, st)) != hipSuccess)
        return e;
    } else {
      if ((e = hipEventRecord(ts.join, ts.stream)) != hipSuccess) return e;
      if ((e = hipStreamWaitEvent(st, ts.join, 0)) != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// A tiled shared expert whose GEMM1 has fewer tiles than the device has CUs
// (a few hundred to a few thousand tokens) runs on a side stream forked from
// st (an event records st's position, the side stream waits on it) and
// joined back at the end (st waits on an event recorded after the shared
// launches), so it overlaps the routed experts instead of running alone on
// part of the device.  The fork comes at the start of the routed GEMM2 stage
// (for fp8 before h is quantised, which the shared GEMM1 then overlaps):
// the routed GEMM1, the longer of the two, keeps the whole device, and the
// shared expert runs beside the routed GEMM2 (measured against forking at
// the start: decode256 2.825 -> 2.766 ms, decode256_fp8 1.537 -> 1.522 ms,
// clustered2048_fp8 2.715 -> 2.675 ms).  Both write disjoint rows of h and
// separate outputs.  A skinny shared expert (T <= kSkinnyRows) streams
// weights like the routed skinny kernels and one that fills the device is
// compute-bound like the routed tiles: both stay on st, where running beside
// the routed kernels would only add contention.
template <int DT>
hipError_t run_ffn(const moe_cfg& c, const Args& a, hipStream_t st, bool planned, bool fork) {
  if (!a.has_shared || a.halves || a.shared_tiled) return run_routed<DT>(c, a, st, planned, fork);
  if (!fork) {
    hipError_t e = run_shared<DT>(c, a, st);
    return e != hipSuccess ? e : run_routed<DT>(c, a, st, planned, false);
  }
  moe::SideStream side;
  hipError_t e = moe::side_stream(&side);
  if (e != hipSuccess) return e;
  // (in units of 256 x 256 output tiles, whatever the kernels' tile widths)
  const long long shared_tiles1 =
      (long long)(a.mid_rest ? c.T / kTileRows + moe::ceil_div(c.T % kTileRows, kMidRows) : moe::ceil_div(c.T, kTileRows)) *
      moe::ceil_div(c.I, kTN / 2);
  if (c.T <= kSkinnyRows || shared_tiles1 >= side.cus) {
    e = run_shared<DT>(c, a, st);
    return e != hipSuccess ? e : run_routed<DT>(c, a, st, planned, true);
  }
  hipError_t es = hipSuccess;
  auto fork_at = [&](int at) -> hipError_t {   // at 2: the routed GEMM2 stage is next
    if (at != 2) return hipSuccess;
    hipError_t ef = hipEventRecord(side.fork, st);
    if (ef == hipSuccess) ef = hipStreamWaitEvent(side.stream, side.fork, 0);
    if (ef != hipSuccess) return ef;
    es = run_shared<DT>(c, a, side.stream);
    return es;
  };
  hipError_t er = run_routed<DT>(c, a, st, planned, true, fork_at);
  // join even after a failed launch, so that work queued later on st never
  // runs ahead of work already queued on the side stream
  if ((e = hipEventRecord(side.join, side.stream)) == hipSuccess) e = hipStreamWaitEvent(st, side.join, 0);
  return es != hipSuccess ? es : er != hipSuccess ? er : e;
}

}  // namespace

namespace moe {

// Capacity of the 256-row tile list: at most P / 256 full tiles, plus one
// partial tile per routed group, plus the shared expert's ceil(T / 256) tiles
// when they join the list.
int ffn_fat_cap(const moe_cfg& c) { return c.T * c.k / kTileRows + c.E + c.T / kTileRows + 1; }

size_t ffn_plan_ints(const moe_cfg& c) {
  const int G = c.E + (c.I_shared > 0 ? 1 : 0);
  // three skinny lists of up to 2G entries (halves); 128-row tiles: at most one per routed group
  return kPlanHead + 6 * (size_t)G + 2 * (size_t)ffn_fat_cap(c) + 2 * (size_t)c.E;
}

PlanArgs ffn_plan_args(const moe_cfg& c, int32_t* plan) {
  PlanArgs p;
  p.plan = plan;
  p.E = c.E;
  p.G = c.E + (c.I_shared > 0 ? 1 : 0);
  p.T = c.T;
  p.fat_cap = ffn_fat_cap(c);
  p.halves = c.T <= 16 ? 1 : 0;
  p.mid_rest = c.w_dtype == MOE_FP8_E4M3 ? 1 : 0;   // HBM-bound medium groups: deeper pipeline on 128-row tiles
  p.shared_tiled = c.I_shared > 0 && c.w_dtype != MOE_FP8_E4M3 && c.T > kSkinnyRows &&
                   (long long)moe::ceil_div(c.T, kTileRows) * moe::ceil_div(c.I, kTN / 2) >= kSharedInListTiles;
  return p;
}

size_t ffn_h_elem_bytes(const moe_cfg& c) { return c.w_dtype == MOE_BF16 ? 2 : 4; }

hipError_t launch_expert_ffn(const moe_cfg& c, const void* x, const int32_t* offsets,
                             const int32_t* sorted_pair, const moe_weights& w, void* y_sorted,
                             void* y_shared, const FfnWs& ws, hipStream_t st, bool planned, bool fork,
                             bool down_only) {
  Args a{};
  a.first_mode = down_only ? 2 : 1;
  if (down_only) fork = false;
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
  a.wsr_shift = c.w_dtype == MOE_FP8_E4M3 && c.w_block_rows == 128 ? 7 : 0;
  a.h = static_cast<uint8_t*>(ws.h);
  a.y_sorted = static_cast<uint8_t*>(y_sorted);
  a.y_shared = static_cast<uint8_t*>(y_shared);
  const PlanArgs pa = ffn_plan_args(c, ws.plan);
  a.plan = pa.plan;
  a.G = pa.G;
  a.fat_cap = pa.fat_cap;
  a.halves = pa.halves;
  a.mid_rest = pa.mid_rest;
  a.shared_tiled = pa.shared_tiled;
  // fp8: the routed tiles quantise their rows of h in GEMM1's epilogue when
  // tiled groups are expected (a mean of more than 16 rows per routed
  // expert), and a launch over the streaming groups' rows does the rest
  // (clustered2048_fp8 2.444 -> 2.417 ms).  Otherwise (decode: groups of a
  // few rows) one vectorised launch over all rows is faster (decode256_fp8
  // +0.5% with the per-group launch), and any tile writes h.
  a.tile_quant = c.w_dtype == MOE_FP8_E4M3 && c.T > kSkinnyRows && !pa.halves && a.P / c.E > kSkinnyRows / 2;
  if (c.w_dtype == MOE_FP8_E4M3) {
    if (!down_only) {
      hipError_t e = launch_quant_fp8(c.T, c.H, c.quant_block, x, MOE_BF16, ws.xq, ws.xs, st);
      if (e != hipSuccess) return e;
    }
    a.a1 = ws.xq;
    a.a1s = ws.xs;
    a.a2 = ws.hq;
    a.a2s = ws.hs;
    return run_ffn<MOE_FP8_E4M3>(c, a, st, planned, fork);
  }
  a.a1 = static_cast<const uint8_t*>(x);
  a.a2 = a.h;
  if (c.w_dtype == MOE_BF16) return run_ffn<MOE_BF16>(c, a, st, planned, fork);
  return run_ffn<MOE_F32>(c, a, st, planned, fork);
}

}  // namespace moe
