// C ABI of the MoE-layer forward: argument validation (always before any
// launch), workspace carving and error reporting.  The stages themselves live
// in route.hip, dispatch.hip, quant.hip, ffn.hip and combine.hip.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/moe.h"
#include <mutex>
#include <new>

#include "moe_launch.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

int hip_fail(hipError_t e, const char* stage) {
  return fail(MOE_ERR_HIP, "%s: %s", stage, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define NEED_PTR(p)                                                               \
  do {                                                                            \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", #p);       \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", #p); \
  } while (0)

constexpr long long kMaxPairs = 1LL << 24;

int check_cfg(const moe_cfg* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %d < 0", c->T);
  if (c->H <= 0 || c->E <= 0 || c->I <= 0) return fail(MOE_ERR_INVALID_ARG, "H, E and I must be positive");
  if (c->k < 1 || c->k > c->E) return fail(MOE_ERR_INVALID_ARG, "k = %d outside [1, E = %d]", c->k, c->E);
  if (c->score != MOE_SCORE_SOFTMAX && c->score != MOE_SCORE_SIGMOID)
    return fail(MOE_ERR_INVALID_ARG, "unknown score function %d", c->score);
  if (!isfinite(c->routed_scale)) return fail(MOE_ERR_INVALID_ARG, "routed_scale is not finite");
  if (c->I_shared < 0) return fail(MOE_ERR_INVALID_ARG, "I_shared < 0");
  if ((long long)c->T * c->k > kMaxPairs) return fail(MOE_ERR_UNSUPPORTED, "T*k above %lld pairs", kMaxPairs);
  if (c->E > 256) return fail(MOE_ERR_UNSUPPORTED, "E = %d > 256", c->E);
  if (c->k > 32) return fail(MOE_ERR_UNSUPPORTED, "k = %d > 32", c->k);
  if (c->I_shared != 0 && c->I_shared != c->I)
    return fail(MOE_ERR_UNSUPPORTED, "shared-expert width %d differs from I = %d", c->I_shared, c->I);
  if (c->n_group < 1 || c->topk_group < 1 || c->topk_group > c->n_group)
    return fail(MOE_ERR_INVALID_ARG, "need 1 <= topk_group (%d) <= n_group (%d)", c->topk_group, c->n_group);
  if (c->n_group > 1) {
    if (c->E % c->n_group) return fail(MOE_ERR_INVALID_ARG, "E = %d not a multiple of n_group = %d", c->E, c->n_group);
    const int gs = c->E / c->n_group;
    if (gs < 2) return fail(MOE_ERR_INVALID_ARG, "groups of one expert have no two-key score");
    if (c->k > c->topk_group * gs)
      return fail(MOE_ERR_INVALID_ARG, "k = %d above the %d experts of %d groups", c->k, c->topk_group * gs, c->topk_group);
    if (c->n_group > 64) return fail(MOE_ERR_UNSUPPORTED, "n_group = %d > 64", c->n_group);
  }
  const bool f32 = c->act_dtype == MOE_F32 && c->w_dtype == MOE_F32;
  const bool bf16 = c->act_dtype == MOE_BF16 && c->w_dtype == MOE_BF16;
  const bool fp8 = c->act_dtype == MOE_BF16 && c->w_dtype == MOE_FP8_E4M3;
  if (!(f32 || bf16 || fp8))
    return fail(MOE_ERR_UNSUPPORTED, "dtype pair act %d / weights %d", c->act_dtype, c->w_dtype);
  if (c->H % 128) return fail(MOE_ERR_UNSUPPORTED, "H = %d not a multiple of 128", c->H);
  if (c->I % 64) return fail(MOE_ERR_UNSUPPORTED, "I = %d not a multiple of 64", c->I);
  if (fp8) {
    if (c->quant_block != 128) return fail(MOE_ERR_UNSUPPORTED, "fp8 block %d != 128", c->quant_block);
    if (c->I % 128) return fail(MOE_ERR_UNSUPPORTED, "fp8 needs I %% 128 == 0");
    if (c->w_block_rows != 1 && c->w_block_rows != 128)
      return fail(MOE_ERR_UNSUPPORTED, "fp8 weight scale blocks of %d rows (1 or 128)", c->w_block_rows);
  }
  return MOE_OK;
}

struct Layout {
  size_t ctr, route_part, seg, plan, h, hq, hs, xq, xs;
  size_t f_idx, f_w, f_counts, f_offsets, f_sorted, f_slot, f_ysorted, f_yshared;
  size_t total;
};

Layout layout(const moe_cfg& c) {
  Layout L{};
  if (c.T == 0) return L;   // no tokens: no call touches the workspace
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~(size_t)255;
    return at;
  };
  const size_t T = c.T, H = c.H, E = c.E, I = c.I, P = T * c.k;
  const size_t Ts = c.I_shared > 0 ? T : 0;
  const bool fp8 = c.w_dtype == MOE_FP8_E4M3;
  const size_t qb = fp8 ? (size_t)c.quant_block : 1;
  L.ctr = take(moe::kRouteCounters * sizeof(int32_t));   // offset 0: must start zeroed
  L.route_part = take(moe::route_ws_bytes(c));
  L.seg = take(moe::dispatch_ws_bytes(c));
  L.plan = take(moe::ffn_plan_ints(c) * sizeof(int32_t));
  L.h = take((P + Ts) * I * moe::ffn_h_elem_bytes(c));
  L.hq = take(fp8 ? (P + Ts) * I : 0);
  L.hs = take(fp8 ? (P + Ts) * (I / qb) * 4 : 0);
  L.xq = take(fp8 ? T * H : 0);
  L.xs = take(fp8 ? T * (H / qb) * 4 : 0);
  L.f_idx = take(P * 4);
  L.f_w = take(P * 4);
  L.f_counts = take(E * 4);
  L.f_offsets = take((E + 1) * 4);
  L.f_sorted = take(P * 4);
  L.f_slot = take(P * 4);
  const size_t ab = c.act_dtype == MOE_F32 ? 4 : 2;
  L.f_ysorted = take(P * H * ab);
  L.f_yshared = take(Ts * H * ab);
  L.total = off;
  return L;
}

int check_ws(const moe_cfg& c, void* ws, size_t ws_bytes, Layout* L) {
  *L = layout(c);
  if (ws_bytes < L->total)
    return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", ws_bytes, L->total);
  if (L->total && ws == nullptr) return fail(MOE_ERR_INVALID_ARG, "ws is NULL");
  if (!aligned16(ws)) return fail(MOE_ERR_INVALID_ARG, "ws is not 16-byte aligned");
  return MOE_OK;
}

int check_weights(const moe_cfg& c, const moe_weights* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  NEED_PTR(w->w13);
  NEED_PTR(w->w2);
  const bool fp8 = c.w_dtype == MOE_FP8_E4M3;
  if (fp8) {
    NEED_PTR(w->w13_scale);
    NEED_PTR(w->w2_scale);
  }
  if (c.I_shared > 0) {
    NEED_PTR(w->ws13);
    NEED_PTR(w->ws2);
    if (fp8) {
      NEED_PTR(w->ws13_scale);
      NEED_PTR(w->ws2_scale);
    }
  }
  return MOE_OK;
}

template <class T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<uint8_t*>(ws) + off);
}

moe::FfnWs ffn_ws(void* ws, const Layout& L) {
  moe::FfnWs f;
  f.plan = at<int32_t>(ws, L.plan);
  f.h = at<void>(ws, L.h);
  f.hq = at<uint8_t>(ws, L.hq);
  f.hs = at<float>(ws, L.hs);
  f.xq = at<uint8_t>(ws, L.xq);
  f.xs = at<float>(ws, L.xs);
  return f;
}

}  // namespace

namespace moe {
void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
}
}  // namespace moe

extern "C" {

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
    default: return "MOE_ERR_UNKNOWN";
  }
}

const char* moe_last_error(void) { return g_err; }

size_t moe_workspace_bytes(const moe_cfg* cfg) {
  if (check_cfg(cfg)) return 0;
  ok();
  const size_t total = layout(*cfg).total;
  return total > 0 ? total : 256;   // never 0 for a valid layer (0 means invalid)
}

int moe_workspace_size(const moe_cfg* cfg, size_t* bytes) {
  int s = check_cfg(cfg);
  if (s) return s;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout(*cfg).total;
  return ok();
}

int moe_workspace_ffn_h(const moe_cfg* cfg, size_t* h_offset, size_t* hq_offset, size_t* hs_offset) {
  int s = check_cfg(cfg);
  if (s) return s;
  if (!h_offset || !hq_offset || !hs_offset) return fail(MOE_ERR_INVALID_ARG, "an offset pointer is NULL");
  const Layout L = layout(*cfg);
  const bool any = cfg->T > 0, fp8 = any && cfg->w_dtype == MOE_FP8_E4M3;
  *h_offset = any ? L.h : SIZE_MAX;
  *hq_offset = fp8 ? L.hq : SIZE_MAX;
  *hs_offset = fp8 ? L.hs : SIZE_MAX;
  return ok();
}

int moe_route(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias, int32_t* topk_idx,
              float* topk_w, void* ws, size_t ws_bytes, void* hip_stream) {
  int s = check_cfg(cfg);
  if (s) return s;
  if (cfg->T == 0) return ok();
  NEED_PTR(x);
  NEED_PTR(w_gate);
  NEED_PTR(topk_idx);
  NEED_PTR(topk_w);
  if (sel_bias && !aligned16(sel_bias)) return fail(MOE_ERR_INVALID_ARG, "sel_bias is not 16-byte aligned");
  Layout L;
  if ((s = check_ws(*cfg, ws, ws_bytes, &L))) return s;
  hipError_t e = moe::launch_route(*cfg, x, w_gate, sel_bias, topk_idx, topk_w, at<float>(ws, L.route_part),
                                   at<int32_t>(ws, L.ctr), static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? ok() : hip_fail(e, "moe_route");
}

int moe_dispatch(const moe_cfg* cfg, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pair, int32_t* pair_slot, void* ws, size_t ws_bytes, void* hip_stream) {
  int s = check_cfg(cfg);
  if (s) return s;
  if (cfg->T == 0) return ok();
  NEED_PTR(topk_idx);
  NEED_PTR(counts);
  NEED_PTR(offsets);
  NEED_PTR(sorted_pair);
  NEED_PTR(pair_slot);
  Layout L;
  if ((s = check_ws(*cfg, ws, ws_bytes, &L))) return s;
  hipError_t e = moe::launch_dispatch(*cfg, topk_idx, counts, offsets, sorted_pair, pair_slot,
                                      at<int32_t>(ws, L.seg), static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? ok() : hip_fail(e, "moe_dispatch");
}

int moe_routing_stats(const moe_cfg* cfg, const int32_t* topk_idx, int32_t n_ranks, int32_t* counts,
                      int32_t* rank_load, float* skew, int32_t* affinity, void* hip_stream) {
  int s = check_cfg(cfg);
  if (s) return s;
  if (n_ranks < 1 || cfg->E % n_ranks)
    return fail(MOE_ERR_INVALID_ARG, "n_ranks = %d does not divide E = %d", n_ranks, cfg->E);
  if (cfg->T == 0) return ok();
  NEED_PTR(topk_idx);
  hipError_t e = moe::launch_routing_stats(*cfg, topk_idx, n_ranks, counts, rank_load, skew, affinity,
                                           static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? ok() : hip_fail(e, "moe_routing_stats");
}

int moe_quantize_fp8(int32_t rows, int32_t cols, int32_t block, const void* in, int32_t in_dtype, uint8_t* codes,
                     float* scales, void* hip_stream) {
  if (rows < 0 || cols < 0) return fail(MOE_ERR_INVALID_ARG, "negative shape");
  if (block <= 0 || block > 256 || block % 64) return fail(MOE_ERR_UNSUPPORTED, "block %d not in {64,128,192,256}", block);
  if (cols % block) return fail(MOE_ERR_INVALID_ARG, "cols %d not a multiple of block %d", cols, block);
  if (in_dtype != MOE_BF16 && in_dtype != MOE_F32) return fail(MOE_ERR_UNSUPPORTED, "input dtype %d", in_dtype);
  if (rows == 0 || cols == 0) return ok();
  NEED_PTR(in);
  NEED_PTR(codes);
  NEED_PTR(scales);
  hipError_t e = moe::launch_quant_fp8(rows, cols, block, in, in_dtype, codes, scales,
                                       static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? ok() : hip_fail(e, "moe_quantize_fp8");
}

namespace {

int expert_ffn_call(const moe_cfg* cfg, const void* x, const int32_t* offsets, const int32_t* sorted_pair,
                    const moe_weights* w, void* y_sorted, void* y_shared, void* ws, size_t ws_bytes,
                    void* hip_stream, bool down_only) {
  const char* what = down_only ? "moe_expert_ffn_down" : "moe_expert_ffn";
  int s = check_cfg(cfg);
  if (s) return s;
  if (cfg->T == 0) return ok();
  if (!down_only) NEED_PTR(x);
  NEED_PTR(offsets);
  NEED_PTR(sorted_pair);
  NEED_PTR(y_sorted);
  if ((s = check_weights(*cfg, w))) return s;
  if (cfg->I_shared > 0) {
    NEED_PTR(y_shared);
  } else if (y_shared) {
    return fail(MOE_ERR_INVALID_ARG, "y_shared given but the layer has no shared expert");
  }
  Layout L;
  if ((s = check_ws(*cfg, ws, ws_bytes, &L))) return s;
  hipError_t e = moe::launch_expert_ffn(*cfg, x, offsets, sorted_pair, *w, y_sorted, y_shared, ffn_ws(ws, L),
                                        static_cast<hipStream_t>(hip_stream), false, true, down_only);
  return e == hipSuccess ? ok() : hip_fail(e, what);
}

}  // namespace

int moe_expert_ffn(const moe_cfg* cfg, const void* x, const int32_t* offsets, const int32_t* sorted_pair,
                   const moe_weights* w, void* y_sorted, void* y_shared, void* ws, size_t ws_bytes,
                   void* hip_stream) {
  return expert_ffn_call(cfg, x, offsets, sorted_pair, w, y_sorted, y_shared, ws, ws_bytes, hip_stream, false);
}

int moe_expert_ffn_down(const moe_cfg* cfg, const int32_t* offsets, const int32_t* sorted_pair,
                        const moe_weights* w, void* y_sorted, void* y_shared, void* ws, size_t ws_bytes,
                        void* hip_stream) {
  return expert_ffn_call(cfg, nullptr, offsets, sorted_pair, w, y_sorted, y_shared, ws, ws_bytes, hip_stream,
                         true);
}

int moe_combine(const moe_cfg* cfg, const void* y_sorted, const void* y_shared, const int32_t* pair_slot,
                const float* topk_w, void* y, void* hip_stream) {
  int s = check_cfg(cfg);
  if (s) return s;
  if (cfg->T == 0) return ok();
  NEED_PTR(y_sorted);
  NEED_PTR(pair_slot);
  NEED_PTR(topk_w);
  NEED_PTR(y);
  if (y_shared && !aligned16(y_shared)) return fail(MOE_ERR_INVALID_ARG, "y_shared is not 16-byte aligned");
  hipError_t e = moe::launch_combine(*cfg, y_sorted, y_shared, pair_slot, topk_w, y,
                                     static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? ok() : hip_fail(e, "moe_combine");
}

}  // extern "C"

namespace {

// Validation of moe_forward's arguments other than the workspace.
int check_forward_args(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias,
                       const moe_weights* w, void* y, int32_t* topk_idx_out, float* topk_w_out,
                       int32_t* counts_out) {
  NEED_PTR(x);
  NEED_PTR(w_gate);
  NEED_PTR(y);
  if (sel_bias && !aligned16(sel_bias)) return fail(MOE_ERR_INVALID_ARG, "sel_bias is not 16-byte aligned");
  if ((topk_idx_out && !aligned16(topk_idx_out)) || (topk_w_out && !aligned16(topk_w_out)) ||
      (counts_out && !aligned16(counts_out)))
    return fail(MOE_ERR_INVALID_ARG, "routing output pointers must be 16-byte aligned");
  return check_weights(*cfg, w);
}

// The whole layer on a validated workspace laid out as L.  With fork = false
// every launch stays on hip_stream (no side stream is created or used).
int forward_on(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias, const moe_weights* w,
               void* y, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* ws, const Layout& L,
               void* hip_stream, bool fork) {
  hipStream_t st = static_cast<hipStream_t>(hip_stream);
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.f_idx);
  float* wt = topk_w_out ? topk_w_out : at<float>(ws, L.f_w);
  int32_t* counts = counts_out ? counts_out : at<int32_t>(ws, L.f_counts);
  int32_t* offsets = at<int32_t>(ws, L.f_offsets);
  int32_t* sorted = at<int32_t>(ws, L.f_sorted);
  int32_t* slot = at<int32_t>(ws, L.f_slot);
  void* ys = at<void>(ws, L.f_ysorted);
  void* ysh = cfg->I_shared > 0 ? at<void>(ws, L.f_yshared) : nullptr;
  hipError_t e = moe::launch_route(*cfg, x, w_gate, sel_bias, idx, wt, at<float>(ws, L.route_part),
                                   at<int32_t>(ws, L.ctr), st);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/route");
  const moe::FfnWs fws = ffn_ws(ws, L);
  const moe::PlanArgs pa = moe::ffn_plan_args(*cfg, fws.plan);
  bool planned = false;   // the dispatch also builds the FFN plan
  e = moe::launch_dispatch(*cfg, idx, counts, offsets, sorted, slot, at<int32_t>(ws, L.seg), st, &pa, &planned);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/dispatch");
  e = moe::launch_expert_ffn(*cfg, x, offsets, sorted, *w, ys, ysh, fws, st, planned, fork);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/expert_ffn");
  e = moe::launch_combine(*cfg, ys, ysh, slot, wt, y, st);
  if (e != hipSuccess) return hip_fail(e, "moe_forward/combine");
  return ok();
}

// Device scratch of moe_forward_noalloc: one copy per GPU, held from the
// module's load until the process ends, zero at load.  In host code
// `scratch` is only a host-side stand-in for the symbol; its device address
// comes from hipGetSymbolAddress, once per device, and only that address is
// ever handed to kernels.
constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "moe_forward_noalloc/device");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "moe_forward_noalloc/hipGetSymbolAddress");
    if (!p) return fail(MOE_ERR_HIP, "moe_forward_noalloc: no device address for the scratch array");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_forward(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias, const moe_weights* w,
                void* y, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* ws, size_t ws_bytes,
                void* hip_stream) {
  int s = check_cfg(cfg);
  if (s) return s;
  if (cfg->T == 0) return ok();
  if ((s = check_forward_args(cfg, x, w_gate, sel_bias, w, y, topk_idx_out, topk_w_out, counts_out))) return s;
  Layout L;
  if ((s = check_ws(*cfg, ws, ws_bytes, &L))) return s;
  return forward_on(cfg, x, w_gate, sel_bias, w, y, topk_idx_out, topk_w_out, counts_out, ws, L, hip_stream, true);
}

int moe_forward_noalloc(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias,
                        const moe_weights* w, void* y, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                        void* hip_stream) {
  int s = check_cfg(cfg);
  if (s) return s;
  if (cfg->T == 0) return ok();
  if ((s = check_forward_args(cfg, x, w_gate, sel_bias, w, y, topk_idx_out, topk_w_out, counts_out))) return s;
  const Layout L = layout(*cfg);
  if (L.total > kScratchBytes)
    return fail(MOE_ERR_WORKSPACE, "moe_forward_noalloc: this layer needs %zu bytes of scratch, above the fixed %zu",
                L.total, kScratchBytes);
  void* ws = nullptr;
  if ((s = scratch_on_current_device(&ws))) return s;
  return forward_on(cfg, x, w_gate, sel_bias, w, y, topk_idx_out, topk_w_out, counts_out, ws, L, hip_stream, false);
}

struct moe_graph {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

int moe_graph_capture(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias,
                      const moe_weights* w, void* y, int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out,
                      void* ws, size_t ws_bytes, void* hip_stream, moe_graph** out) {
  if (!out) return fail(MOE_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (cfg && cfg->T == 0) return fail(MOE_ERR_INVALID_ARG, "T = 0: nothing to capture");
  // One eager call: validates the arguments and creates the per-device
  // state that is made on first use (side stream, kernel attributes).
  int s = moe_forward(cfg, x, w_gate, sel_bias, w, y, topk_idx_out, topk_w_out, counts_out, ws, ws_bytes, hip_stream);
  if (s) return s;
  hipStream_t cs;
  hipError_t e = moe::capture_stream(&cs);
  if (e != hipSuccess) return hip_fail(e, "moe_graph_capture/stream");
  if ((e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal)) != hipSuccess)
    return hip_fail(e, "moe_graph_capture/begin");
  s = moe_forward(cfg, x, w_gate, sel_bias, w, y, topk_idx_out, topk_w_out, counts_out, ws, ws_bytes, cs);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  if (s || e != hipSuccess) {
    if (g) (void)hipGraphDestroy(g);
    return s ? s : hip_fail(e, "moe_graph_capture/end");
  }
  hipGraphExec_t ex = nullptr;
  if ((e = hipGraphInstantiate(&ex, g, nullptr, nullptr, 0)) != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(e, "moe_graph_capture/instantiate");
  }
  *out = new (std::nothrow) moe_graph{g, ex};
  if (!*out) {
    (void)hipGraphExecDestroy(ex);
    (void)hipGraphDestroy(g);
    return fail(MOE_ERR_HIP, "moe_graph_capture: out of host memory");
  }
  return ok();
}

int moe_graph_launch(const moe_graph* g, void* hip_stream) {
  if (!g) return fail(MOE_ERR_INVALID_ARG, "graph is NULL");
  hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(hip_stream));
  return e == hipSuccess ? ok() : hip_fail(e, "moe_graph_launch");
}

int moe_graph_destroy(moe_graph* g) {
  if (!g) return ok();
  hipError_t e1 = hipGraphExecDestroy(g->exec);
  hipError_t e2 = hipGraphDestroy(g->graph);
  delete g;
  if (e1 != hipSuccess) return hip_fail(e1, "moe_graph_destroy");
  return e2 == hipSuccess ? ok() : hip_fail(e2, "moe_graph_destroy");
}

}  // extern "C"
