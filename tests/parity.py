"""Comparison rules shared by the GPU parity tests and the bench's parity line.

Outputs (floating point): e_i = |g_i - o_i| / max(|o_i|, rms(o)) must stay
within ELEM_TOL[dtype] for every element, and ||g - o||_F / ||o||_F within
FROB_TOL[dtype].  bf16 and fp8 bounds are the ones the layer is specified to;
the fp32 bound is derived from fp32 accumulation over K <= 8192 terms
(sqrt(K) * 2^-24 * a few, with margin).

Routing: expert indices must match exactly on every token whose fp64 keys
have no adjacent gap below NEAR_TIE among the first k+1 sorted keys; near-tie
tokens are counted, and their GPU choice must be a valid top-k within the gap.
"""

import numpy as np
import torch

ELEM_TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
FROB_TOL = {"f32": 1e-5, "bf16": 5e-3, "fp8": 5e-3}
WEIGHT_RTOL = 1e-4
NEAR_TIE = 1e-6


def tol_key(cfg) -> str:
    return "fp8" if cfg.w_dtype == "fp8" else cfg.act_dtype


def to_np(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().to("cpu")
        if t.dtype in (torch.bfloat16, torch.float16, torch.float32):
            t = t.to(torch.float64)
        return t.numpy()
    return np.asarray(t)


def output_errors(gpu, ref):
    g = to_np(gpu).astype(np.float64)
    o = np.asarray(ref, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    if o.size == 0:
        return 0.0, 0.0
    rms = float(np.sqrt(np.mean(o * o)))
    floor = max(rms, 1e-300)
    elem = float(np.max(np.abs(g - o) / np.maximum(np.abs(o), floor)))
    fro = float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))
    return elem, fro


def assert_outputs_close(gpu, ref, key, what="output"):
    elem, fro = output_errors(gpu, ref)
    assert elem <= ELEM_TOL[key] and fro <= FROB_TOL[key], (
        f"{what}: max elementwise rel err {elem:.3e} (tol {ELEM_TOL[key]}), "
        f"Frobenius rel err {fro:.3e} (tol {FROB_TOL[key]})")
    return elem, fro


def compare_routing(gpu_idx, gpu_w, oracle_route, k):
    """Returns (n_near_tie, mismatched_tokens).  Asserts exact indices on
    non-near-tie tokens and weights within WEIGHT_RTOL where indices agree.
    A token is a near tie when two of its first k+1 eligible keys, or (with
    group-limited routing) the last chosen and the first unchosen group
    scores, lie within NEAR_TIE; there the GPU's choice must be a valid one."""
    gi = to_np(gpu_idx).astype(np.int64)
    gw = to_np(gpu_w).astype(np.float64)
    oi = oracle_route["idx"]
    near_g = oracle_route["group_gap"] < NEAR_TIE
    near = (oracle_route["gap"] < NEAR_TIE) | near_g
    same = (gi == oi).all(axis=1)
    bad = np.nonzero(~same & ~near)[0]
    assert len(bad) == 0, f"{len(bad)} tokens route differently without a near tie, first {bad[:8]}"
    elig = oracle_route["elig"]
    for t in np.nonzero(near & ~same)[0]:
        assert len(set(gi[t].tolist())) == k
        if near_g[t]:
            # groups: each chosen expert's group scores within NEAR_TIE of the
            # last chosen group; at most topk_group groups
            gsc = oracle_route["group_scores"][t]
            ng, tg = oracle_route["n_group"], oracle_route["topk_group"]
            gs = len(elig[t]) // ng
            last = np.sort(gsc)[::-1][tg - 1]
            groups = set((gi[t] // gs).tolist())
            assert len(groups) <= tg and all(gsc[g] >= last - NEAR_TIE for g in groups), f"token {t}: invalid groups"
            continue
        chosen = elig[t, gi[t]]
        kth = np.sort(elig[t])[::-1][k - 1]
        assert chosen.min() >= kth - NEAR_TIE, f"token {t}: invalid near-tie choice"
        assert np.all(np.diff(chosen) <= NEAR_TIE)
    if same.any():
        np.testing.assert_allclose(gw[same], oracle_route["w"][same], rtol=WEIGHT_RTOL, atol=0)
    return int(near.sum()), np.nonzero(~same)[0]
