/*
 * moe.h -- C ABI of the MoE-layer forward on one AMD Instinct MI355X (gfx950).
 *
 * The layer (DeepSeek-V3/R1 style), as stated in Perplexity's "Lower latency
 * and higher throughput with multi-node DeepSeek deployment", section
 * "Expert parallelism": every token is sent to k *different* routed experts,
 * their outputs are summed with weights, and the output of one shared expert,
 * which every token also goes through, is added.  The router is, after the
 * vLLM DeepSeek-V4.1-Flash article (section "Kernels", item "Mega-Gate"),
 * gate GEMM -> expert scoring -> bias -> top-k.  Dense per-expert execution
 * needs the routing aggregated per expert (Perplexity, section "MoE
 * router"), and every kernel reads the per-expert token counts on the device
 * instead of syncing them to the host (Perplexity, section "Quantization",
 * paragraph on the MoE router under CUDA graphs).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller; the layer's
 *   calls never allocate device memory, free it or synchronise.  State kept
 *   between calls: a thread-local error string; per host thread and device,
 *   two side streams with their events and a capture stream, made on first
 *   use; per (kernel, device), whether its LDS limit was raised; and the
 *   measurement state of moe_profile_start/stop.  Arrays are dense row-major.
 * - Work is enqueued on `hip_stream` (a hipStream_t; NULL = default stream)
 *   and the call returns; faults inside kernels surface at the caller's next
 *   synchronisation.  No call reads device memory on the host.
 * - Every argument is validated on the host BEFORE anything is enqueued: a
 *   call that returns an error has launched nothing and written nothing.
 * - T == 0 returns MOE_OK and enqueues nothing.
 * - "Pairs": p = t*k + j is the j-th chosen expert of token t; P = T*k.
 * - Weight matrices are [out_features, in_features] row-major.
 * - The library never prints, throws across the ABI or aborts.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null required pointer, bad shape, k out of range, misaligned */
  MOE_ERR_UNSUPPORTED = 2, /* valid layer the kernels do not implement (listed per field) */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4          /* a HIP launch failed; moe_last_error() has the detail */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Expert scoring applied to the gate logits (a reading of "expert scoring"):
 * softmax over all E experts, or an elementwise sigmoid. */
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

typedef struct {
  int32_t T;           /* tokens, >= 0 */
  int32_t H;           /* hidden size; multiple of 128 */
  int32_t E;           /* routed experts in this call, 1..256 */
  int32_t k;           /* experts per token, 1..min(E, 32) */
  int32_t I;           /* routed-expert intermediate size; multiple of 64 (quant_block for FP8) */
  int32_t I_shared;    /* shared-expert intermediate size: 0 (none) or I */
  int32_t score;       /* moe_score */
  int32_t act_dtype;   /* x, gate weight and y: MOE_F32 or MOE_BF16 */
  int32_t w_dtype;     /* expert weights: MOE_F32 (with act F32), MOE_BF16 (act BF16),
                          MOE_FP8_E4M3 (act BF16) */
  int32_t quant_block; /* FP8 block width along K: 128; ignored otherwise */
  float routed_scale;  /* multiplies the renormalised combine weights (1.0) */
  int32_t n_group;     /* group-limited routing (Perplexity, "Lower latency and higher throughput with
                          multi-node DeepSeek deployment", section "MoE router": Mixtral routing is the
                          DeepSeek routing whose group holds all experts).  The E experts form n_group
                          groups of E / n_group consecutive experts; a group's score is the sum of its
                          two largest selection keys (score + bias; the pages give no group score, this
                          is the DeepSeek-V3 reading); the top-k runs over the experts of the topk_group
                          best groups (ties to the lower group).  n_group = 1 or topk_group = n_group:
                          plain top-k.  Needs E % n_group == 0, E / n_group >= 2, n_group <= 64
                          (UNSUPPORTED above), 1 <= topk_group <= n_group and
                          k <= topk_group * E / n_group (INVALID_ARG otherwise). */
  int32_t topk_group;  /* groups kept eligible per token */
  int32_t w_block_rows; /* FP8 weight scale blocks: 1 (one scale per row per quant_block columns)
                           or 128 (128 x 128 tiles, Perplexity, "Quantization"); ignored otherwise */
} moe_cfg;

/* Expert weights.  Routed: w13 [E, 2I, H] (rows [0,I) = gate projection W1,
 * rows [I,2I) = up projection W3), w2 [E, H, I].  Shared: ws13 [2I, H],
 * ws2 [H, I] (NULL when I_shared == 0).  For MOE_FP8_E4M3 the *_scale arrays
 * hold one fp32 scale per block of w_block_rows rows x quant_block columns
 * ([.., rows / w_block_rows, cols / 128]); the value of weight (r, c) is
 * e4m3(code) * scale[r / w_block_rows][c / 128].  Scales are NULL otherwise. */
typedef struct {
  const void* w13;
  const float* w13_scale;
  const void* w2;
  const float* w2_scale;
  const void* ws13;
  const float* ws13_scale;
  const void* ws2;
  const float* ws2_scale;
} moe_weights;

/* Human-readable name of a moe_status value (static string). */
const char* moe_status_str(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Bytes of device workspace that every call below needs for this layer: an
 * upper bound independent of the routing, so that one allocation serves
 * every batch of this shape (the graph-per-batch-size rule of Perplexity,
 * "Lower latency and higher throughput with multi-node DeepSeek
 * deployment", section "Quantization", MoE-router paragraph).  Returns 0
 * when cfg is invalid (moe_last_error() says why); a valid layer always
 * needs more than 0 bytes.
 * The workspace's first 256 bytes hold the router's completion counters:
 * they must be zero before a workspace is first used (zero-fill it once
 * after allocating it), and every call leaves them zero again.  The rest
 * needs no initialisation. */
size_t moe_workspace_bytes(const moe_cfg* cfg);

/* The same bound through an out-parameter, returning a moe_status (the form
 * every other entry point uses). */
int moe_workspace_size(const moe_cfg* cfg, size_t* bytes);

/* Where the expert FFNs leave their intermediate in the workspace: the
 * SwiGLU output h = SiLU(a W1^T) * (a W3^T) of every row (Perplexity,
 * "GroupGEMM"), and for fp8 weights its per-row block quantisation, which
 * the down projection reads (same article, "Quantization").  h has P + T
 * rows of I (P = T * k): row s < offsets[E] is pair sorted_pair[s]'s, in
 * dispatch order; rows P .. P + T - 1 are the shared expert's when
 * I_shared > 0.  Other rows are unspecified.  With fp8 weights the codes
 * and scales are what the down projection reads; h itself is then scratch
 * (routed groups of more than 32 rows quantise their rows inside GEMM1 and
 * never write them to h).
 *   h_offset   byte offset of h: bf16 for bf16 weights, fp32 otherwise
 *   hq_offset  fp8 weights: byte offset of h's E4M3 codes [P + T, I]
 *   hs_offset  fp8 weights: byte offset of their fp32 scales
 *              [P + T, I / quant_block]
 * hq_offset and hs_offset are SIZE_MAX unless the weights are fp8; all three
 * are SIZE_MAX when T == 0.  The contents are those of the last
 * moe_expert_ffn or moe_forward on the workspace, once it has completed.
 * Returns MOE_ERR_INVALID_ARG for a NULL pointer, or cfg's error. */
int moe_workspace_ffn_h(const moe_cfg* cfg, size_t* h_offset, size_t* hq_offset, size_t* hs_offset);

/* Router (steps: gate GEMM, scoring, selection bias, top-k, weights; the
 * vLLM DeepSeek-V4.1-Flash article, section "Kernels", item "Mega-Gate").
 * Below 512 bf16 tokens (up to 1024 fp32 tokens) it is one launch:
 * the last workgroup to finish a 16-token tile's partial gate GEMM sums the
 * partials and selects, using the workspace's counters (see
 * moe_workspace_bytes). */
/* Router arguments:
 *   x        [T, H] act_dtype          w_gate [E, H] act_dtype
 *   sel_bias [E] fp32 or NULL: added to the scores for choosing experts only
 *   topk_idx [T, k] int32 out: chosen experts, descending biased score,
 *            equal scores ordered by the lower expert index
 *   topk_w   [T, k] fp32 out: unbiased scores of the chosen experts divided
 *            by their sum, times routed_scale
 * Logits accumulate in fp32 in a fixed order (bitwise reproducible). */
int moe_route(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias,
              int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* hip_stream);

/* Dispatch: per-expert aggregation of the routing (Perplexity, "MoE router").
 *   topk_idx    [T, k] int32 in: each token's k experts, which must be
 *               distinct (a token goes to k *different* experts, section
 *               "Expert parallelism") and in [0, E).  An id outside [0, E)
 *               is skipped: it is counted nowhere, its pair gets
 *               pair_slot = -1 and moe_combine adds nothing for it.  With
 *               repeated ids a group can exceed T rows; moe_expert_ffn
 *               then leaves some y_sorted rows unwritten (no access goes
 *               out of bounds, but the output is unspecified).
 *   counts      [E] int32 out: pairs routed to each expert
 *   offsets     [E+1] int32 out: exclusive running sum, offsets[E] = number
 *               of pairs with a valid id (T*k when all are valid)
 *   sorted_pair [T*k] int32 out: for each expert, its pair ids in ascending
 *               order, at positions offsets[e] .. offsets[e+1]-1
 *   pair_slot   [T*k] int32 out: inverse permutation (sorted_pair[pair_slot[p]] = p),
 *               -1 for a skipped pair
 * Bitwise deterministic. */
int moe_dispatch(const moe_cfg* cfg, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                 int32_t* sorted_pair, int32_t* pair_slot, void* ws, size_t ws_bytes,
                 void* hip_stream);

/* Per-row block quantisation to OCP FP8 E4M3 (Perplexity, "Quantization":
 * activations get one scale per 128-element block, computed on the fly).
 *   in     [rows, cols] MOE_BF16 or MOE_F32 (in_dtype); cols % block == 0
 *   codes  [rows, cols] uint8 out; scales [rows, cols/block] fp32 out
 * scale = fp32(amax/448) (1 for an all-zero block); code = e4m3 of
 * fp32(v/scale), round to nearest even, saturating at +-448. */
int moe_quantize_fp8(int32_t rows, int32_t cols, int32_t block, const void* in, int32_t in_dtype,
                     uint8_t* codes, float* scales, void* hip_stream);

/* Expert FFNs: every routed expert's SwiGLU over its dispatched rows (a
 * grouped GEMM; Perplexity, "GroupGEMM"), and the shared expert over all T
 * rows.  SwiGLU(a) = (SiLU(a W1^T) * (a W3^T)) W2^T.  For FP8 weights, x and
 * the SwiGLU output are block-quantised per row per quant_block first.
 * Accumulation is fp32; outputs are rounded once to act_dtype.
 *   x           [T, H] act_dtype; offsets / sorted_pair from moe_dispatch
 *   y_sorted    [T*k, H] act_dtype out: row s = expert output of pair sorted_pair[s]
 *   y_shared    [T, H] act_dtype out (NULL iff I_shared == 0)
 * Per-expert row counts are read on the device (no host sync). */
int moe_expert_ffn(const moe_cfg* cfg, const void* x, const int32_t* offsets,
                   const int32_t* sorted_pair, const moe_weights* w, void* y_sorted,
                   void* y_shared, void* ws, size_t ws_bytes, void* hip_stream);

/* The expert FFNs' down projection alone (Perplexity, "GroupGEMM": the
 * second grouped GEMM, y = h W2^T per group, and the shared expert's): the
 * y_sorted and y_shared that moe_expert_ffn would write, computed from the h
 * the workspace holds where moe_workspace_ffn_h places it, instead of from
 * x.  The caller writes h there first, in that row layout; for fp8 weights
 * the E4M3 codes and fp32 scales of h, which are used as they are (not
 * requantised).  Other arguments as moe_expert_ffn.  For callers that
 * produce h themselves, and to test the down projection on its own. */
int moe_expert_ffn_down(const moe_cfg* cfg, const int32_t* offsets, const int32_t* sorted_pair,
                        const moe_weights* w, void* y_sorted, void* y_shared, void* ws, size_t ws_bytes,
                        void* hip_stream);

/* Combine (Perplexity, "Lower latency and higher throughput with multi-node
 * DeepSeek deployment", section "Expert parallelism": the outputs of a
 * token's k routed experts are summed with weights, and the shared expert's
 * output, which every token also goes through, is added):
 *   y[t] = y_shared[t] + sum_j topk_w[t,j] * y_sorted[pair_slot[t*k+j]],
 * accumulated in fp32 in the order shared, j = 0..k-1 (deterministic);
 * pairs with pair_slot < 0 (skipped by moe_dispatch) add nothing.
 *   y_sorted [T*k, H] and y_shared [T, H] (may be NULL: treated as 0) in
 *   act_dtype; y [T, H] act_dtype out. */
int moe_combine(const moe_cfg* cfg, const void* y_sorted, const void* y_shared,
                const int32_t* pair_slot, const float* topk_w, void* y, void* hip_stream);

/* The whole layer (Perplexity, "Lower latency and higher throughput with
 * multi-node DeepSeek deployment", section "Expert parallelism": k weighted
 * routed experts plus the shared expert per token; the router's steps are
 * those of the vLLM DeepSeek-V4.1-Flash article, section "Kernels", item
 * "Mega-Gate"): route -> dispatch -> expert FFN -> combine, enqueued on
 * hip_stream (the shared expert and, when both FFN regimes occur, the tiled
 * groups may run on library side streams forked from and joined back to it).
 *   y [T, H] act_dtype out.  topk_idx_out [T,k], topk_w_out [T,k] and
 *   counts_out [E] are optional copies of the routing (NULL to skip). */
int moe_forward(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias,
                const moe_weights* w, void* y, int32_t* topk_idx_out, float* topk_w_out,
                int32_t* counts_out, void* ws, size_t ws_bytes, void* hip_stream);

/* moe_forward for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * kernels as moe_forward, with the same arguments except the workspace:
 * the intermediates live in a fixed device scratch array inside the library
 * (64 MiB, one per GPU, held from the library's load until the process
 * ends), so the call allocates nothing and calls no allocating routine.
 * Every launch stays on hip_stream (no side stream).  Layers whose
 * workspace exceeds the scratch (moe_workspace_bytes(cfg) > 64 MiB; e.g.
 * the 8192-token prefill share) return MOE_ERR_WORKSPACE before anything
 * is enqueued.  All calls on one GPU share its scratch: calls that overlap
 * in time on one GPU (two host threads, or two streams not ordered by the
 * caller) race and give undefined results.  The router's counters at the
 * start of the scratch are zero when the library loads and every call
 * leaves them zero; the rest of the scratch needs no initialisation. */
int moe_forward_noalloc(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias,
                        const moe_weights* w, void* y, int32_t* topk_idx_out, float* topk_w_out,
                        int32_t* counts_out, void* hip_stream);

/* Graph of one whole-layer call (Perplexity, "Lower latency and higher
 * throughput with multi-node DeepSeek deployment", section "Quantization",
 * MoE-router paragraph: one graph is captured per batch size, so the
 * kernels read the per-expert token counts on the device).
 * moe_graph_capture first runs moe_forward once on hip_stream (validating
 * the arguments exactly as moe_forward does, writing its outputs, and
 * creating the per-device state made on first use), then captures the same
 * call on a private stream and instantiates it.  The graph keeps the
 * pointers it was captured with: each moe_graph_launch runs the whole layer
 * on the current contents of x, w_gate, sel_bias and the weights, into the
 * same y / routing outputs / workspace, on hip_stream (ordered like any
 * other work on it).  Routings may differ between launches; T, the shapes
 * and the buffers may not.  Launches of one graph must not overlap (they
 * share the workspace).  Capture allocates the graph (host and device
 * resources); launch allocates nothing.  *out is NULL on failure; T = 0 is
 * INVALID_ARG.  Do not capture while moe_profile_start() is on. */
typedef struct moe_graph moe_graph;
int moe_graph_capture(const moe_cfg* cfg, const void* x, const void* w_gate, const float* sel_bias,
                      const moe_weights* w, void* y, int32_t* topk_idx_out, float* topk_w_out,
                      int32_t* counts_out, void* ws, size_t ws_bytes, void* hip_stream, moe_graph** out);
int moe_graph_launch(const moe_graph* g, void* hip_stream);
int moe_graph_destroy(moe_graph* g);   /* NULL is a no-op */

/* Routing statistics of one batch (the GRACE-MoE summary in the pages:
 * section "Expert Grouping" builds an expert affinity matrix from activation
 * patterns, section "Expert Replication" the load skew rho = W_max / W_mean
 * of the group loads).  Groups are n_ranks ranges of E / n_ranks consecutive
 * experts (expert-parallel ranks).
 *   topk_idx   [T, k] int32 (from moe_route); entries outside [0, E) are skipped
 *   counts     [E] int32 out: pairs routed to each expert (NULL to skip)
 *   rank_load  [n_ranks] int32 out: pairs routed to each rank's experts (NULL to skip)
 *   skew       [2] fp32 out: {max rank load, max expert load} divided by the
 *              mean load T*k/n_ranks, T*k/E; 0 when T*k = 0 (NULL to skip)
 *   affinity   [E, E] int32 out: tokens routed to both i and j; the diagonal
 *              holds counts (NULL to skip)
 * Needs 1 <= n_ranks, E % n_ranks == 0 (INVALID_ARG).  Integer results are
 * exact and order-independent; T = 0 enqueues nothing and leaves the outputs
 * untouched.  No workspace. */
int moe_routing_stats(const moe_cfg* cfg, const int32_t* topk_idx, int32_t n_ranks, int32_t* counts,
                      int32_t* rank_load, float* skew, int32_t* affinity, void* hip_stream);

/* ---- Per-kernel timing (measurement tools; not part of the layer).
 * Between moe_profile_start(only) and moe_profile_stop(), every kernel the
 * library launches (or, when `only` is not NULL, every kernel of that name)
 * is bracketed by two HIP events recorded on the stream it is launched on.  moe_profile_stop() waits for those events and returns, per
 * kernel name, the launch count and the summed event-to-event time; entries
 * beyond max_entries are dropped (*n_entries still counts them).  Events are
 * pooled by the library and reused.  Do not enable while capturing a graph.
 * Process-wide state, guarded by a mutex. */
typedef struct {
  char name[48];
  int32_t launches;
  double total_ms;
} moe_kernel_time;

int moe_profile_start(const char* only);
int moe_profile_stop(moe_kernel_time* out, int32_t max_entries, int32_t* n_entries);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
