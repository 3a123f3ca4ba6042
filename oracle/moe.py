"""The MoE-layer forward written out as its definition, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).  Slow on purpose: every
stage is the plain statement of what it computes, with no blocking, fusion
or reordering.

Pages (cited by title and section):

* [PPLX] Perplexity, "Lower latency and higher throughput with multi-node
  DeepSeek deployment" (Japanese and Arabic copies).
  - "Expert parallelism": 256 routed experts and one shared expert; every
    token goes to 8 *different* routed experts whose outputs are summed with
    weights, and through the shared expert, whose output is added.
  - "MoE router": the router is a sort that also tracks the indices of the
    sorted elements (top-k); dense dispatch/combine needs the routing
    information aggregated per expert instead of per token.
  - "Quantization": fp8 weights and per-128 activation blocks; the SiLU
    (SwiGLU) kernel with block quantisation of its output.
  - "Roofline" / "GroupGEMM": group i multiplies [m_i, k] x [k, n].
* [VLLM] vLLM article on DeepSeek-V4.1-Flash optimisations, section
  "Kernels", item "Mega-Gate": the router is gate GEMM, expert scoring, bias
  and top-k selection.

Readings where the pages are silent (each is listed in the design notes):
scores are softmax over all experts or elementwise sigmoid; the selection
bias is added to the scores for choosing experts only and the combine
weights are the unbiased scores of the chosen experts renormalised to sum to
one (routed scale 1); equal keys are ordered by lower expert index; the
chosen experts are listed in descending key order; pairs inside an expert's
segment are in ascending pair id p = t*k + j; no capacity limit, no dropping;
one shared expert shaped like a routed one; SwiGLU is
``SiLU(x W1^T) * (x W3^T)`` followed by ``W2``; in the fp8 layer x and the
SwiGLU output h are block-quantised per row per 128 before their GEMMs.
"""

from dataclasses import dataclass
from typing import Callable, Optional, Tuple

import numpy as np

from .fp8 import dequantize_weight, quantize_rows_fp8


def to_f64(t) -> np.ndarray:
    """Exact conversion of a torch tensor (any device, f32/bf16) or array to fp64."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu").to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


# --------------------------------------------------------------------------- router

def route(x, wg, bias, k: int, score: str, routed_scale: float = 1.0, n_group: int = 1, topk_group: int = 1):
    """Gate GEMM -> expert scoring -> selection bias -> top-k -> weights.

    [VLLM] "Mega-Gate" names the four steps; [PPLX] "Expert parallelism"
    requires k different experts per token and a weighted sum.

    Group-limited routing ([PPLX] "MoE router": the router is shared by all
    MoE models, Mixtral routing being the DeepSeek routing whose group holds
    all experts).  With n_group > 1 the E experts form n_group groups of
    E / n_group consecutive experts; a group's score is the sum of its two
    largest selection keys; the topk_group groups of highest score (ties to
    the lower group) stay eligible and the top-k runs over their experts
    only.  The pages give no group scores, so the two-largest-keys sum is the
    DeepSeek-V3 reading; n_group = 1 (or topk_group = n_group) is plain top-k.

    Returns a dict with ``logits`` [T,E], ``scores`` [T,E], ``keys`` [T,E],
    ``idx`` int64 [T,k] (descending key, ties to the lower expert),
    ``w`` [T,k], ``gap`` [T]: the smallest difference between adjacent keys
    among the first min(k+1, E) sorted eligible keys (a small gap marks a near
    tie), ``group_gap`` [T]: the score difference between the last chosen
    and the first unchosen group (inf without a group stage), ``elig`` [T,E]:
    the keys with the experts of unchosen groups at -inf, and
    ``group_scores`` [T, n_group] (None without a group stage).
    """
    x = np.asarray(x, dtype=np.float64)
    wg = np.asarray(wg, dtype=np.float64)
    T, E = x.shape[0], wg.shape[0]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    logits = x @ wg.T
    if score == "softmax":
        z = logits - logits.max(axis=1, keepdims=True)
        ez = np.exp(z)
        scores = ez / ez.sum(axis=1, keepdims=True)
    elif score == "sigmoid":
        scores = 1.0 / (1.0 + np.exp(-logits))
    else:
        raise ValueError(f"unknown scoring {score!r}")
    keys = scores + (0.0 if bias is None else np.asarray(bias, dtype=np.float64)[None, :])
    elig = keys
    group_gap = np.full(T, np.inf)
    gscore = None
    if n_group > 1:
        gs = E // n_group
        if gs * n_group != E or gs < 2 or not 1 <= topk_group <= n_group or k > topk_group * gs:
            raise ValueError("need E = n_group * g with g >= 2, 1 <= topk_group <= n_group, k <= topk_group * g")
        top2 = np.sort(keys.reshape(T, n_group, gs), axis=2)[:, :, -2:]
        gscore = top2[:, :, 0] + top2[:, :, 1]
        gorder = np.argsort(-gscore, axis=1, kind="stable")       # equal scores: lower group first
        chosen = np.zeros((T, n_group), dtype=bool)
        np.put_along_axis(chosen, gorder[:, :topk_group], True, axis=1)
        elig = np.where(np.repeat(chosen, gs, axis=1), keys, -np.inf)
        if topk_group < n_group:
            gsorted = np.take_along_axis(gscore, gorder, axis=1)
            group_gap = gsorted[:, topk_group - 1] - gsorted[:, topk_group]
    # A stable sort of the negated keys lists equal keys by ascending index.
    order = np.argsort(-elig, axis=1, kind="stable")
    idx = order[:, :k]
    nk = min(k + 1, E)
    ks = np.take_along_axis(elig, order[:, :nk], axis=1)
    with np.errstate(invalid="ignore"):
        gap = (ks[:, :-1] - ks[:, 1:]).min(axis=1) if nk > 1 else np.full(T, np.inf)
    gap = np.where(np.isnan(gap), np.inf, gap)
    sel = np.take_along_axis(scores, idx, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True) * routed_scale
    return dict(logits=logits, scores=scores, keys=keys, elig=elig, idx=idx, w=w, gap=gap,
                group_gap=group_gap, group_scores=gscore, n_group=n_group, topk_group=topk_group)


# --------------------------------------------------------------------------- dispatch

def dispatch(idx, E: int):
    """Per-expert aggregation of the routing ([PPLX] "MoE router").

    counts[e] = number of pairs routed to e; offsets = exclusive running sum
    (offsets[E] = T*k); sorted_pair lists, expert by expert, the pair ids
    p = t*k + j routed to that expert in ascending order; pair_slot is its
    inverse.  Written as plain loops over the pairs.
    """
    flat = np.asarray(idx, dtype=np.int64).reshape(-1)
    P = flat.shape[0]
    counts = np.zeros(E, dtype=np.int64)
    for p in range(P):
        counts[flat[p]] += 1
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:E].copy()
    sorted_pair = np.empty(P, dtype=np.int64)
    pair_slot = np.empty(P, dtype=np.int64)
    for p in range(P):
        e = flat[p]
        s = fill[e]
        sorted_pair[s] = p
        pair_slot[p] = s
        fill[e] += 1
    return dict(counts=counts, offsets=offsets, sorted_pair=sorted_pair, pair_slot=pair_slot)


# --------------------------------------------------------------------------- experts

@dataclass
class OracleWeights:
    """fp64 expert weights, produced one expert at a time.

    ``expert(e)`` and ``shared()`` return (W1 [I,H], W3 [I,H], W2 [H,I]); the
    fp8 variants are dequantised as code value times the scale of its
    block_rows x 128 block (1 x 128 or 128 x 128).
    """
    E: int
    expert: Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]
    shared: Optional[Callable[[], Tuple[np.ndarray, np.ndarray, np.ndarray]]]
    fp8: bool
    block: int = 128

    @staticmethod
    def from_inputs(inp) -> "OracleWeights":
        cfg = inp.cfg
        fp8 = cfg.w_dtype == "fp8"
        blk = cfg.quant_block
        brows = getattr(cfg, "w_block_rows", 1)

        def split(w13, w2, s13=None, s2=None):
            if fp8:
                w13f = dequantize_weight(w13.cpu().numpy(), s13.cpu().numpy(), blk, brows)
                w2f = dequantize_weight(w2.cpu().numpy(), s2.cpu().numpy(), blk, brows)
            else:
                w13f, w2f = to_f64(w13), to_f64(w2)
            i = w13f.shape[0] // 2
            return w13f[:i], w13f[i:], w2f

        def expert(e):
            return split(inp.w13[e], inp.w2[e],
                         inp.w13_scale[e] if fp8 else None, inp.w2_scale[e] if fp8 else None)

        shared = None
        if inp.ws13 is not None:
            def shared():
                return split(inp.ws13, inp.ws2, inp.ws13_scale, inp.ws2_scale)
        return OracleWeights(cfg.E, expert, shared, fp8, blk)


def swiglu_hidden(a, w1, w3):
    """One expert's SwiGLU output h = SiLU(a W1^T) * (a W3^T), SiLU(z) = z sigmoid(z)."""
    a = np.asarray(a, dtype=np.float64)
    g = a @ w1.T
    u = a @ w3.T
    return g / (1.0 + np.exp(-g)) * u


def swiglu_ffn(a, w1, w3, w2, quant_h: bool = False, block: int = 128):
    """One expert: h = SiLU(a W1^T) * (a W3^T); y = h W2^T.

    With ``quant_h`` the SwiGLU output is block-quantised per row per
    ``block`` before the down projection ([PPLX] "Quantization", SiLU kernel).
    """
    h = swiglu_hidden(a, w1, w3)
    if quant_h:
        h = quantize_rows_fp8(h, block)[2]
    return h @ w2.T


def prepare_activations(x, fp8: bool, block: int = 128):
    """The expert GEMMs' input: x itself, or x block-quantised per token per
    128 and dequantised (the fp8 layer; [PPLX] "Quantization")."""
    x = np.asarray(x, dtype=np.float64)
    return quantize_rows_fp8(x, block)[2] if fp8 else x


def expert_ffn(xa, offsets, sorted_pair, k: int, weights: OracleWeights):
    """Grouped SwiGLU over the dispatched rows ([PPLX] "GroupGEMM": group e
    multiplies its m_e gathered rows by expert e's weights) plus the shared
    expert over all T rows ([PPLX] "Expert parallelism").

    ``xa`` is the output of ``prepare_activations``.  Returns (y_sorted [P,H]
    in dispatch order, y_shared [T,H]; zeros when there is no shared expert).
    """
    xa = np.asarray(xa, dtype=np.float64)
    T, H = xa.shape
    P = int(offsets[-1])
    y_sorted = np.zeros((P, H))
    for e in range(weights.E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue
        rows = np.asarray(sorted_pair[lo:hi]) // k
        w1, w3, w2 = weights.expert(e)
        y_sorted[lo:hi] = swiglu_ffn(xa[rows], w1, w3, w2, weights.fp8, weights.block)
    y_shared = np.zeros((T, H))
    if weights.shared is not None:
        w1, w3, w2 = weights.shared()
        y_shared = swiglu_ffn(xa, w1, w3, w2, weights.fp8, weights.block)
    return y_sorted, y_shared


# --------------------------------------------------------------------------- routing statistics

def routing_stats(idx, E: int, n_ranks: int):
    """Per-expert load, load skew and the expert affinity matrix of one batch.

    The GRACE-MoE summary in the pages (section "Expert Grouping") builds an
    expert affinity matrix A from activation patterns and drives replication
    by the load skew rho = W_max / W_mean of the group loads (section "Expert
    Replication").  Readings: A[i][j] is the number of tokens routed to both
    experts i and j (A = M^T M for the T x E routing incidence matrix M, so
    the diagonal holds the per-expert loads); the groups are n_ranks equal
    ranges of consecutive experts (expert-parallel ranks).  Written as plain
    loops over tokens and expert pairs.

    Returns counts [E], rank_load [n_ranks], rho_rank, rho_expert (the skew
    with one group per expert) and affinity [E, E] (int64).
    """
    idx = np.asarray(idx, dtype=np.int64)
    T, k = idx.shape
    if E % n_ranks:
        raise ValueError("need E divisible by n_ranks")
    counts = np.zeros(E, dtype=np.int64)
    affinity = np.zeros((E, E), dtype=np.int64)
    for t in range(T):
        for a in range(k):
            counts[idx[t, a]] += 1
            for b in range(k):
                affinity[idx[t, a], idx[t, b]] += 1
    per = E // n_ranks
    rank_load = np.zeros(n_ranks, dtype=np.int64)
    for r in range(n_ranks):
        for e in range(r * per, (r + 1) * per):
            rank_load[r] += counts[e]
    P = T * k
    rho_rank = rank_load.max() / (P / n_ranks) if P else 0.0
    rho_expert = counts.max() / (P / E) if P else 0.0
    return dict(counts=counts, rank_load=rank_load, rho_rank=float(rho_rank), rho_expert=float(rho_expert),
                affinity=affinity)


# --------------------------------------------------------------------------- combine

def combine(y_sorted, y_shared, pair_slot, w, k: int):
    """y[t] = y_shared[t] + sum_j w[t,j] * y_sorted[pair_slot[t*k+j]]
    ([PPLX] "Expert parallelism": weighted sum of the routed outputs plus the
    shared expert's output)."""
    w = np.asarray(w, dtype=np.float64)
    T = w.shape[0]
    y = np.array(y_shared, dtype=np.float64, copy=True)
    for t in range(T):
        for j in range(k):
            y[t] += w[t, j] * y_sorted[int(pair_slot[t * k + j])]
    return y


# --------------------------------------------------------------------------- whole layer

def forward(inp, weights: Optional[OracleWeights] = None):
    """The whole layer for every token, stage by stage, with intermediates."""
    cfg = inp.cfg
    weights = weights or OracleWeights.from_inputs(inp)
    x = to_f64(inp.x)
    r = route(x, to_f64(inp.wg), to_f64(inp.bias), cfg.k, cfg.score,
              n_group=cfg.n_group, topk_group=cfg.topk_group)
    d = dispatch(r["idx"], cfg.E)
    xa = prepare_activations(x, weights.fp8, weights.block)
    y_sorted, y_shared = expert_ffn(xa, d["offsets"], d["sorted_pair"], cfg.k, weights)
    y = combine(y_sorted, y_shared, d["pair_slot"], r["w"], cfg.k)
    return dict(route=r, dispatch=d, xa=xa, y_sorted=y_sorted, y_shared=y_shared, y=y)


def forward_tokens(inp, tokens, weights: Optional[OracleWeights] = None, workers: int = 1):
    """The layer's output for the listed tokens only, token by token.

    Routing, activation quantisation and the expert FFNs act on each token on
    its own, so y[t] = sum_j w[t,j] FFN_{idx[t,j]}(x[t]) + FFN_shared(x[t])
    ([PPLX] "Expert parallelism") is computed without any dispatch.  Each
    touched expert's weights are converted once for all listed tokens.
    With ``workers`` > 1 the touched experts are evaluated on that many
    threads; their outputs are still added in ascending expert order, so the
    result is the same bits either way.
    Returns (y [n,H], route dict for the listed tokens).
    """
    cfg = inp.cfg
    weights = weights or OracleWeights.from_inputs(inp)
    tokens = np.asarray(tokens, dtype=np.int64)
    x = to_f64(inp.x[tokens.tolist()]) if len(tokens) else np.zeros((0, cfg.H))
    r = route(x, to_f64(inp.wg), to_f64(inp.bias), cfg.k, cfg.score,
              n_group=cfg.n_group, topk_group=cfg.topk_group)
    xa = prepare_activations(x, weights.fp8, weights.block)
    y = np.zeros_like(xa)

    def one_expert(e):
        rows, js = np.nonzero(r["idx"] == e)
        w1, w3, w2 = weights.expert(int(e))
        return rows, js, swiglu_ffn(xa[rows], w1, w3, w2, weights.fp8, weights.block)

    experts = [int(e) for e in np.unique(r["idx"])]
    if workers > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(workers) as ex:
            outs = list(ex.map(one_expert, experts))
    else:
        outs = map(one_expert, experts)
    for rows, js, ye in outs:                      # ascending expert order
        y[rows] += r["w"][rows, js][:, None] * ye
    if weights.shared is not None:
        w1, w3, w2 = weights.shared()
        y += swiglu_ffn(xa, w1, w3, w2, weights.fp8, weights.block)
    return y, r
