"""Pins of the fp64 oracle against things other than itself.

Every test here is CPU-only.  The pins are: hand-derived worked cases
(tests/golden/, each with its derivation), brute force over all expert
subsets, library routines for special cases (numpy's bincount / stable
argsort, torch's float8 cast and dense linear layers), closed forms, and
invariants of the layer.  They are chosen so that a dropped term, a wrong
sign or index, or a swapped operand in the oracle fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.fp8 import _MAGS, dequantize_weight
from moe_inputs import get_config, make_inputs

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _weights_from_arrays(w1, w3, w2, shared=None):
    E = len(w1)
    return oracle.OracleWeights(
        E, lambda e: (np.asarray(w1[e], float), np.asarray(w3[e], float), np.asarray(w2[e], float)),
        (lambda: tuple(np.asarray(a, float) for a in shared)) if shared is not None else None,
        fp8=False)


# ----------------------------------------------------------------- worked cases

def test_worked_sigmoid_case(golden_dir):
    g = _load(golden_dir, "worked_sigmoid_T1_E4_k2.json")
    wts = _weights_from_arrays(g["w1"], g["w3"], g["w2"])
    for case in g["cases"]:
        r = oracle.route(g["x"], g["wg"], case["bias"], g["k"], g["score"])
        assert r["idx"].tolist() == case["idx"]
        np.testing.assert_allclose(r["w"], case["w"], rtol=0, atol=1e-15)
        assert (r["gap"][0] < 1e-6) == case["near_tie"]
        d = oracle.dispatch(r["idx"], g["E"])
        for key in ("counts", "offsets", "sorted_pair", "pair_slot"):
            assert d[key].tolist() == case[key], key
        ys, ysh = oracle.expert_ffn(np.asarray(g["x"]), d["offsets"], d["sorted_pair"], g["k"], wts)
        y = oracle.combine(ys, ysh, d["pair_slot"], r["w"], g["k"])
        np.testing.assert_allclose(y, case["y"], rtol=1e-14, atol=0)


def test_worked_softmax_case(golden_dir):
    g = _load(golden_dir, "worked_softmax_T1_E4_k2.json")
    logits = np.asarray(g["logits"])
    # H = 1, x = [[1]], wg = logits^T: the gate GEMM reproduces the given logits
    r = oracle.route(np.ones((1, 1)), logits.T.copy(), None, g["k"], g["score"])
    np.testing.assert_allclose(r["scores"], g["scores"], rtol=1e-14)
    assert r["idx"].tolist() == g["idx"]
    np.testing.assert_allclose(r["w"], g["w"], rtol=1e-14)


# ----------------------------------------------------------------- router

def _route_keys(keys, k):
    """Route with the given keys as sigmoid scores: x = logit(keys), wg = I."""
    keys = np.asarray(keys, float)
    logits = np.log(keys) - np.log1p(-keys)
    return oracle.route(logits, np.eye(keys.shape[1]), None, k, "sigmoid")


@pytest.mark.parametrize("E,k", [(4, 1), (6, 2), (8, 3), (12, 4), (16, 4)])
def test_topk_brute_force(E, k):
    rng = np.random.default_rng(E * 100 + k)
    for _ in range(20):
        s = rng.uniform(0.01, 0.99, size=(1, E))
        r = _route_keys(s, k)
        # exhaustive search: with distinct keys the top-k set maximises the key sum
        best = max(itertools.combinations(range(E), k), key=lambda c: sum(s[0, list(c)]))
        assert sorted(r["idx"][0].tolist()) == sorted(best)
        # listed in descending key order
        sel = s[0, r["idx"][0]]
        assert np.all(np.diff(sel) < 0)
        # every chosen key beats every other key
        rest = np.setdiff1d(np.arange(E), r["idx"][0])
        if len(rest):
            assert sel.min() > s[0, rest].max()


def test_topk_ties_go_to_lower_index():
    keys = np.array([[0.5, 0.7, 0.5, 0.7, 0.2, 0.5]])
    r = _route_keys(keys, 4)
    assert r["idx"][0].tolist() == [1, 3, 0, 2]
    assert r["gap"][0] == 0.0


def test_bias_selects_but_does_not_weight():
    rng = np.random.default_rng(3)
    T, H, E, k = 32, 16, 12, 3
    x, wg = rng.normal(size=(T, H)), rng.normal(size=(E, H)) / 4
    bias = rng.uniform(-0.3, 0.3, size=E)
    r = oracle.route(x, wg, bias, k, "sigmoid")
    sig = 1 / (1 + np.exp(-(x @ wg.T)))
    for t in range(T):
        brute = max(itertools.combinations(range(E), k), key=lambda c: sum(sig[t, list(c)] + bias[list(c)]))
        assert sorted(r["idx"][t].tolist()) == sorted(brute)
    # weights come from the unbiased scores of the chosen experts
    sel = np.take_along_axis(sig, r["idx"], 1)
    np.testing.assert_allclose(r["w"], sel / sel.sum(1, keepdims=True), rtol=1e-13)
    # a constant bias changes nothing
    r0 = oracle.route(x, wg, None, k, "sigmoid")
    rc = oracle.route(x, wg, np.full(E, 0.05), k, "sigmoid")
    assert (r0["idx"] == rc["idx"]).all()
    np.testing.assert_allclose(r0["w"], rc["w"], rtol=1e-14)


def test_softmax_weights_equal_softmax_of_chosen_logits():
    rng = np.random.default_rng(5)
    T, H, E, k = 40, 24, 16, 4
    x, wg = rng.normal(size=(T, H)), rng.normal(size=(E, H)) / 5
    r = oracle.route(x, wg, None, k, "softmax")
    lsel = np.take_along_axis(r["logits"], r["idx"], 1)
    ref = torch.softmax(torch.from_numpy(lsel), dim=1).numpy()
    np.testing.assert_allclose(r["w"], ref, rtol=1e-13)
    np.testing.assert_allclose(r["scores"].sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(r["w"].sum(1), 1.0, rtol=1e-14)


# ----------------------------------------------------------------- dispatch

@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 5, 5), (64, 16, 4), (300, 32, 8), (513, 256, 8)])
def test_dispatch_against_numpy(T, E, k):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    d = oracle.dispatch(idx, E)
    flat = idx.reshape(-1)
    np.testing.assert_array_equal(d["counts"], np.bincount(flat, minlength=E))
    np.testing.assert_array_equal(d["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    np.testing.assert_array_equal(d["sorted_pair"], np.argsort(flat, kind="stable"))
    np.testing.assert_array_equal(d["pair_slot"][d["sorted_pair"]], np.arange(T * k))
    # every token appears exactly k times
    np.testing.assert_array_equal(np.bincount(d["sorted_pair"] // k, minlength=T), np.full(T, k))
    assert d["offsets"][-1] == T * k
    assert (np.count_nonzero(d["counts"]) <= min(E, T * k))


def test_dispatch_all_to_one_expert():
    idx = np.zeros((50, 1), dtype=np.int64)
    d = oracle.dispatch(idx, 3)
    assert d["counts"].tolist() == [50, 0, 0]
    assert d["sorted_pair"].tolist() == list(range(50))


# ----------------------------------------------------------------- fp8 codec

def test_e4m3_hand_values(golden_dir):
    g = _load(golden_dir, "e4m3_values.json")
    for v, code in g["encode"]:
        assert int(oracle.e4m3_encode(np.array([v]))[0]) == code, v
    for code, v in g["decode"]:
        assert oracle.e4m3_decode(np.array([code], np.uint8))[0] == v, code


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.e4m3_decode(codes.numpy())
    nan = np.isnan(ref)
    assert (np.isnan(mine) == nan).all()
    np.testing.assert_array_equal(mine[~nan], ref[~nan])


def test_e4m3_encode_matches_torch_and_brute_force():
    rng = np.random.default_rng(11)
    v = np.concatenate([
        rng.normal(size=20000) * 100,
        rng.normal(size=20000) * 1e-2,
        rng.uniform(-600, 600, size=5000),
        (_MAGS[:-1] + _MAGS[1:]) / 2,                 # exact midpoints: ties
        -(_MAGS[:-1] + _MAGS[1:]) / 2,
        _MAGS, -_MAGS, [0.0, 447.9, 448.0, 449.0, 464.0, 479.0, 1e9],
    ]).astype(np.float32).astype(np.float64)
    mine = oracle.e4m3_encode(v)
    ref = torch.from_numpy(np.clip(v, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(mine, ref)
    # brute force on a subset: nearest of all 127 magnitudes, ties to the even code
    for x in v[::97]:
        a = min(abs(x), 448.0)
        d = np.abs(_MAGS - a)
        cands = np.nonzero(d == d.min())[0]
        c = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        assert (int(mine[list(v).index(x)]) & 0x7F) == c


def test_quantize_rows_blocks_and_scales():
    rng = np.random.default_rng(2)
    a = rng.normal(size=(5, 384)) * np.array([1.0, 1e-3, 50.0]).repeat(128)[None, :]
    a[3, 128:256] = 0.0
    codes, scale, deq = oracle.quantize_rows_fp8(a, 128)
    for i in range(5):
        for b in range(3):
            blk = a[i, b * 128:(b + 1) * 128]
            amax = np.abs(blk).max()
            exp_scale = 1.0 if amax == 0 else float(np.float32(amax / 448.0))
            assert scale[i, b] == exp_scale
            # the block's largest magnitude maps to (about) 448
            if amax:
                assert abs(np.abs(deq[i, b * 128:(b + 1) * 128]).max() - amax) <= amax * 2 ** -4
    assert (deq[3, 128:256] == 0).all()
    rel = np.abs(deq - a) / np.maximum(np.abs(a), 1e-300)
    big = np.abs(a) > np.abs(a).reshape(5, 3, 128).max(2).repeat(128, 1) * 2 ** -6
    assert rel[big].max() <= 2 ** -4 + 1e-12          # half an ulp of a 3-bit mantissa


# ----------------------------------------------------------------- expert FFN / layer

def _dense_swiglu_torch(x, w1, w3, w2):
    F = torch.nn.functional
    x, w1, w3, w2 = (torch.from_numpy(np.asarray(t, float)) for t in (x, w1, w3, w2))
    return F.linear(F.silu(F.linear(x, w1)) * F.linear(x, w3), w2).numpy()


def _rand_layer(rng, T, H, E, k, I, shared=True):
    x = rng.normal(size=(T, H))
    wg = rng.normal(size=(E, H)) / math.sqrt(H)
    w1 = rng.normal(size=(E, I, H)) / math.sqrt(H)
    w3 = rng.normal(size=(E, I, H)) / math.sqrt(H)
    w2 = rng.normal(size=(E, H, I)) / math.sqrt(I)
    sh = (rng.normal(size=(I, H)) / math.sqrt(H), rng.normal(size=(I, H)) / math.sqrt(H),
          rng.normal(size=(H, I)) / math.sqrt(I)) if shared else None
    return x, wg, w1, w3, w2, sh


def _layer(x, wg, bias, k, score, wts):
    r = oracle.route(x, wg, bias, k, score)
    d = oracle.dispatch(r["idx"], wts.E)
    ys, ysh = oracle.expert_ffn(x, d["offsets"], d["sorted_pair"], k, wts)
    return oracle.combine(ys, ysh, d["pair_slot"], r["w"], k), r, d, ys, ysh


def test_single_expert_is_dense_swiglu_plus_shared():
    rng = np.random.default_rng(7)
    x, wg, w1, w3, w2, sh = _rand_layer(rng, 9, 32, 1, 1, 16)
    wts = _weights_from_arrays(w1, w3, w2, sh)
    for score in ("sigmoid", "softmax"):
        y, r, *_ = _layer(x, wg, None, 1, score, wts)
        np.testing.assert_allclose(r["w"], 1.0)
        ref = _dense_swiglu_torch(x, w1[0], w3[0], w2[0]) + _dense_swiglu_torch(x, *sh)
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_give_twice_the_shared_output():
    rng = np.random.default_rng(8)
    x, wg, w1, w3, w2, sh = _rand_layer(rng, 33, 24, 10, 3, 8)
    E = 10
    wts = _weights_from_arrays([sh[0]] * E, [sh[1]] * E, [sh[2]] * E, sh)
    y, *_ = _layer(x, wg, rng.uniform(-0.1, 0.1, E), 3, "sigmoid", wts)
    np.testing.assert_allclose(y, 2 * _dense_swiglu_torch(x, *sh), rtol=1e-12, atol=1e-12)


def test_zero_down_projection_and_zero_input():
    rng = np.random.default_rng(9)
    x, wg, w1, w3, w2, sh = _rand_layer(rng, 12, 16, 6, 2, 8)
    wts0 = _weights_from_arrays(w1, w3, np.zeros_like(w2), sh)
    y, r, d, ys, ysh = _layer(x, wg, None, 2, "sigmoid", wts0)
    np.testing.assert_array_equal(y, ysh)
    wts = _weights_from_arrays(w1, w3, w2, sh)
    y0, *_ = _layer(np.zeros_like(x), wg, None, 2, "sigmoid", wts)
    np.testing.assert_array_equal(y0, 0.0)


def test_layer_matches_per_token_formulation():
    rng = np.random.default_rng(10)
    x, wg, w1, w3, w2, sh = _rand_layer(rng, 40, 32, 8, 3, 16)
    wts = _weights_from_arrays(w1, w3, w2, sh)
    bias = rng.uniform(-0.1, 0.1, 8)
    y, r, *_ = _layer(x, wg, bias, 3, "sigmoid", wts)
    # per token, straight from the statement: sum_j w_j FFN_{e_j}(x_t) + FFN_s(x_t)
    for t in range(0, 40, 7):
        ref = _dense_swiglu_torch(x[t:t + 1], *sh)[0]
        for j in range(3):
            e = r["idx"][t, j]
            ref = ref + r["w"][t, j] * _dense_swiglu_torch(x[t:t + 1], w1[e], w3[e], w2[e])[0]
        np.testing.assert_allclose(y[t], ref, rtol=1e-12, atol=1e-13)


def test_forward_and_forward_tokens_agree_on_tiny_workload():
    cfg = get_config("tiny_f32")
    inp = make_inputs(cfg, "cpu")
    full = oracle.forward(inp)
    toks = [0, 5, 17, 63]
    y, r = oracle.forward_tokens(inp, toks)
    np.testing.assert_allclose(y, full["y"][toks], rtol=1e-12, atol=1e-12)
    assert (r["idx"] == full["route"]["idx"][toks]).all()
    # the thread pool over experts changes the scheduling only: same bits
    y4, _ = oracle.forward_tokens(inp, toks, workers=4)
    assert np.array_equal(y, y4)


def test_fp8_activation_quantiser_is_exact_on_representable_blocks():
    """A row whose every 128-block is (block scale) x (e4m3 code values), with
    one element per block at code 0x7E (448), quantises to itself exactly;
    each block has its own scale, so using a wrong block's scale breaks it."""
    rng = np.random.default_rng(12)
    codes = rng.choice(np.arange(0x30, 0x78), size=(4, 384)).astype(np.uint8)
    codes[:, ::128] = 0x7E
    codes[1, 5] |= 0x80                                  # a negative element
    bscale = np.array([0.5, 3.0, 2.0 ** -10])
    x = oracle.e4m3_decode(codes) * np.repeat(bscale, 128)[None, :]
    c2, s2, xa = oracle.quantize_rows_fp8(x, 128)
    np.testing.assert_array_equal(s2, np.tile(bscale, (4, 1)))
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(oracle.prepare_activations(x, True), x)
    # quantising a quantised row again is the identity
    np.testing.assert_array_equal(oracle.prepare_activations(xa, True), xa)


def test_swiglu_quantises_h_per_row_block():
    rng = np.random.default_rng(13)
    I, H = 256, 8
    a = rng.normal(size=(3, H))
    w1 = rng.normal(size=(I, H))
    w3 = rng.normal(size=(I, H))
    w2 = np.zeros((I, I)); np.fill_diagonal(w2, 1.0)        # y = h: exposes h
    h = _dense_swiglu_torch(a, w1, w3, np.eye(I))
    y = oracle.swiglu_ffn(a, w1, w3, w2, quant_h=True)
    ref = oracle.quantize_rows_fp8(h, 128)[2]
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    assert not np.allclose(y, h, rtol=1e-6)                   # quantisation really happened


def test_swiglu_hidden_is_the_dense_gated_product():
    """h alone, against torch's SiLU and linear layers; and y = h W2^T."""
    rng = np.random.default_rng(17)
    I, H = 48, 16
    a = rng.normal(size=(5, H))
    w1, w3 = rng.normal(size=(I, H)), rng.normal(size=(I, H))
    w2 = rng.normal(size=(H, I))
    h = oracle.swiglu_hidden(a, w1, w3)
    np.testing.assert_allclose(h, _dense_swiglu_torch(a, w1, w3, np.eye(I)), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(oracle.swiglu_ffn(a, w1, w3, w2), h @ w2.T, rtol=1e-12, atol=1e-14)
    # the gate, not the up projection, goes through SiLU
    assert not np.allclose(h, oracle.swiglu_hidden(a, w3, w1), rtol=1e-3)


def test_fp8_weights_dequantise_per_row_block():
    cfg = get_config("tiny_f32").with_(w_dtype="fp8", act_dtype="bf16", T=2, E=2, k=1, H=256, I=128)
    inp = make_inputs(cfg, "cpu")
    w1, w3, w2 = oracle.OracleWeights.from_inputs(inp).expert(1)
    raw = inp.w13[1].view(torch.float8_e4m3fn).to(torch.float64)
    sc = inp.w13_scale[1].to(torch.float64).repeat_interleave(128, dim=1)
    ref = (raw * sc).numpy()
    np.testing.assert_array_equal(np.concatenate([w1, w3]), ref)
    np.testing.assert_array_equal(dequantize_weight(inp.w2[1].numpy(), inp.w2_scale[1].numpy()),
                                  (inp.w2[1].view(torch.float8_e4m3fn).to(torch.float64)
                                   * inp.w2_scale[1].to(torch.float64).repeat_interleave(128, 1)).numpy())


# --------------------------------------------------------------------------- group-limited routing

def _sigmoid(v):
    return 1.0 / (1.0 + math.exp(-v))


def test_group_limited_worked_cases(golden_dir):
    """Hand-worked cases (tests/golden/group_limited_E8_G4.json): the group
    score is a two-largest-keys sum of the biased keys, ties go to the lower
    group, the weights use the unbiased scores."""
    g = _load(golden_dir, "group_limited_E8_G4.json")
    for case in g["cases"]:
        logits = np.array(case["logits"])[None, :]
        bias = np.array(case["bias"], dtype=np.float64)
        r = oracle.route(logits, np.eye(8), bias, case["k"], "sigmoid",
                         n_group=case["n_group"], topk_group=case["topk_group"])
        assert r["idx"][0].tolist() == case["idx"], case["name"]
        plain = oracle.route(logits, np.eye(8), bias, case["k"], "sigmoid")
        assert plain["idx"][0].tolist() == case["plain_idx"], case["name"]
        s = [_sigmoid(case["logits"][e]) for e in case["idx"]]
        np.testing.assert_allclose(r["w"][0], np.array(s) / sum(s), rtol=1e-12)
        # the group near-tie gap: last chosen group minus best unchosen group
        assert abs(r["group_gap"][0] - case["group_gap"]) <= 1e-12, case["name"]


def _brute_force_group_route(keys, n_group, topk_group, k):
    """Every topk_group-subset of groups; the one with the largest total of
    group scores (two largest keys each), the lexicographically smallest on
    ties; then the k largest eligible keys, smaller index first on ties."""
    E = len(keys)
    gs = E // n_group
    gscore = []
    for gi in range(n_group):
        best = second = -math.inf
        for e in range(gi * gs, (gi + 1) * gs):
            if keys[e] > best:
                best, second = keys[e], best
            elif keys[e] > second:
                second = keys[e]
        gscore.append(best + second)
    best_set, best_total = None, -math.inf
    for subset in itertools.combinations(range(n_group), topk_group):
        total = sum(gscore[gi] for gi in subset)
        if total > best_total:
            best_set, best_total = subset, total
    elig = [e for e in range(E) if e // gs in best_set]
    return sorted(elig, key=lambda e: (-keys[e], e))[:k], _brute_force_group_gap(gscore, best_set)


def _brute_force_group_gap(gscore, chosen):
    """Smallest chosen group score minus the largest unchosen one (inf when
    every group is chosen): how far the group choice is from a tie."""
    unchosen = [g for g in range(len(gscore)) if g not in chosen]
    if not unchosen:
        return math.inf
    return min(gscore[g] for g in chosen) - max(gscore[g] for g in unchosen)


@pytest.mark.parametrize("E,n_group,topk_group,k", [(8, 4, 2, 3), (12, 3, 1, 2), (16, 4, 3, 5), (16, 8, 2, 4)])
def test_group_limited_matches_brute_force(E, n_group, topk_group, k):
    rng = np.random.default_rng(E * 100 + n_group * 10 + topk_group)
    T, H = 40, 6
    x = rng.standard_normal((T, H))
    wg = rng.standard_normal((E, H))
    bias = rng.uniform(-0.2, 0.2, E)
    r = oracle.route(x, wg, bias, k, "sigmoid", n_group=n_group, topk_group=topk_group)
    keys = 1.0 / (1.0 + np.exp(-(x @ wg.T))) + bias
    for t in range(T):
        idx, gap = _brute_force_group_route(keys[t].tolist(), n_group, topk_group, k)
        assert r["idx"][t].tolist() == idx
        assert abs(r["group_gap"][t] - gap) <= 1e-12, (t, r["group_gap"][t], gap)


def test_group_limited_all_groups_is_plain_topk():
    """topk_group = n_group keeps every expert eligible (the Mixtral case):
    the group stage runs and must change nothing."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((50, 10))
    wg = rng.standard_normal((32, 10))
    bias = rng.uniform(-0.1, 0.1, 32)
    for score in ("sigmoid", "softmax"):
        plain = oracle.route(x, wg, bias, 6, score)
        for n_group in (2, 4, 8, 16):
            r = oracle.route(x, wg, bias, 6, score, n_group=n_group, topk_group=n_group)
            np.testing.assert_array_equal(r["idx"], plain["idx"])
            np.testing.assert_array_equal(r["w"], plain["w"])


def test_group_limited_invariants():
    rng = np.random.default_rng(11)
    E, n_group, topk_group, k = 64, 8, 3, 8
    x = rng.standard_normal((100, 12))
    wg = rng.standard_normal((E, 12))
    r = oracle.route(x, wg, None, k, "sigmoid", n_group=n_group, topk_group=topk_group)
    gs = E // n_group
    for t in range(100):
        groups = set(int(e) // gs for e in r["idx"][t])
        assert len(groups) <= topk_group
        assert len(set(r["idx"][t].tolist())) == k
    assert np.all(r["group_gap"] >= 0)


# --------------------------------------------------------------------------- routing statistics

def test_routing_stats_worked_case(golden_dir):
    g = _load(golden_dir, "routing_stats_T3_E4_k2.json")
    r = oracle.routing_stats(np.array(g["idx"]), g["E"], g["n_ranks"])
    assert r["counts"].tolist() == g["counts"]
    assert r["affinity"].tolist() == g["affinity"]
    assert r["rank_load"].tolist() == g["rank_load"]
    assert r["rho_rank"] == pytest.approx(g["rho_rank"], rel=1e-15)
    assert r["rho_expert"] == pytest.approx(g["rho_expert"], rel=1e-15)


def test_routing_stats_closed_form_and_invariants():
    """A = M^T M for the T x E routing incidence matrix M (a matrix product
    against the oracle's loops); symmetric, diagonal = loads, row sums =
    k * loads, total = T k^2; skews at least 1."""
    rng = np.random.default_rng(5)
    T, E, k, D = 300, 32, 6, 4
    idx = np.argsort(rng.random((T, E)), axis=1)[:, :k]
    r = oracle.routing_stats(idx, E, D)
    M = np.zeros((T, E), dtype=np.int64)
    M[np.arange(T)[:, None], idx] = 1
    A = r["affinity"]
    np.testing.assert_array_equal(A, M.T @ M)
    np.testing.assert_array_equal(A, A.T)
    np.testing.assert_array_equal(np.diag(A), r["counts"])
    np.testing.assert_array_equal(A.sum(axis=1), k * r["counts"])
    assert A.sum() == T * k * k
    np.testing.assert_array_equal(r["rank_load"], r["counts"].reshape(D, -1).sum(axis=1))
    assert r["rho_rank"] >= 1 and r["rho_expert"] >= r["rho_rank"] - 1e-12


def test_routing_stats_balanced_routing_has_unit_skew():
    T, E, k = 64, 16, 4
    idx = (np.arange(T)[:, None] * k + np.arange(k)[None, :]) % E     # every expert k*T/E times
    r = oracle.routing_stats(idx, E, 4)
    assert r["rho_rank"] == 1.0 and r["rho_expert"] == 1.0


# --------------------------------------------------------------------------- 128 x 128 fp8 weight tiles

def test_dequantize_weight_128x128_tiles():
    """Each value is its code (decoded by torch's float8_e4m3fn, a library
    independent of the oracle's table) times the scale of its 128 x 128 tile:
    checked element by element with explicit loops; and 1 x 128 scales that
    repeat a tile's scale on all its rows give the same values."""
    rng = np.random.default_rng(3)
    n, kdim = 256, 384
    codes = rng.integers(0, 256, (n, kdim), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0                    # no NaN codes
    scales = rng.uniform(0.5, 2.0, (n // 128, kdim // 128))
    v = dequantize_weight(codes, scales, 128, 128)
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for r in range(0, n, 7):
        for c in range(kdim):
            assert v[r, c] == dec[r, c] * scales[r // 128, c // 128]
    per_row = np.repeat(scales, 128, axis=0)
    np.testing.assert_array_equal(dequantize_weight(codes, per_row, 128, 1), v)
