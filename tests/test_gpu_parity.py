"""GPU parity: the HIP library, called through its C ABI, against the fp64 oracle.

Inputs are seeded and synthetic (moe_inputs).  Every expected value comes from
oracle/ alone; when a stage is tested on its own, its upstream inputs come
from the oracle (or from the seeded generators), never from the GPU.

Sizes: small layers the oracle finishes in seconds but that still span
several tiles and ragged tails of both expert-FFN regimes; three mid-size
layers whose whole output is checked; and the named workloads at full size:
every token's routing, every token's output for the decode workloads, and
for the prefill share and the clustered fp8 layer the tokens at each
expert's first and last slot and at the tile boundaries, plus whole groups of
every row class and the whole shared-expert output through the expert-FFN
stage on the oracle's dispatch.
"""

import os

import numpy as np
import pytest
import torch

import oracle
import mixture_experts_layer_11_amd as moe
from moe_inputs import CONFIGS, get_config, make_inputs, make_router_inputs
from parity import (assert_outputs_close, compare_routing, output_errors, to_np, tol_key)

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()          # fails loudly when the HIP library is missing


def _log(*a):
    print(*a, flush=True)


# Small layers: several tiles, ragged tails, both FFN regimes.
SMALL = {
    "tiny_f32": get_config("tiny_f32"),
    "small_bf16": get_config("decode16").with_(name="small_bf16", T=200, H=1024, E=32, k=4, I=256, I_shared=256),
    "small_fp8": get_config("clustered2048_fp8").with_(name="small_fp8", T=150, H=512, E=16, k=4, I=256,
                                                      I_shared=256),
    "softmax_e10_f32": get_config("tiny_f32").with_(name="softmax_e10_f32", T=37, E=10, k=3, I=192, I_shared=0),
    "k_eq_E_bf16": get_config("decode16").with_(name="k_eq_E_bf16", T=33, H=256, E=4, k=4, I=128, I_shared=128),
    "one_expert_bf16": get_config("decode16").with_(name="one_expert_bf16", T=70, H=384, E=1, k=1, I=128,
                                                   I_shared=128),
    "one_token_bf16": get_config("decode16").with_(name="one_token_bf16", T=1, H=512, E=64, k=8, I=128,
                                                  I_shared=128),
    # decode-sized shared experts (T <= 32) of each streaming variant, one per dtype
    "t24_bf16": get_config("decode16").with_(name="t24_bf16", T=24, H=512, E=16, k=4, I=256, I_shared=256),
    "t12_fp8": get_config("clustered2048_fp8").with_(name="t12_fp8", T=12, H=512, E=16, k=2, I=256, I_shared=256),
    "t20_f32": get_config("tiny_f32").with_(name="t20_f32", T=20, E=8, k=2),
    # T <= 16: groups of 9..16 rows and the shared expert run as 8-row halves in the <= 8-row launch
    "t16_e4_halves_bf16": get_config("decode16").with_(name="t16_e4_halves_bf16", T=16, H=512, E=4, k=2, I=256,
                                                       I_shared=256),
    # 17..32 tokens: the split-K shared-expert kernel, fp8
    "t20_fp8": get_config("clustered2048_fp8").with_(name="t20_fp8", T=20, H=512, E=16, k=2, I=256, I_shared=256),
    # fp8 weights in 128 x 128 scale tiles: tiled and streaming groups, both shared-expert paths
    "small_fp8_tiles": get_config("decode16_fp8").with_(name="small_fp8_tiles", T=150, H=512, E=16, k=4, I=256,
                                                        I_shared=256),
    "t12_fp8_tiles": get_config("decode16_fp8").with_(name="t12_fp8_tiles", T=12, H=512, E=16, k=2, I=256,
                                                      I_shared=256),
    # fp8 groups of ~150 and ~350 rows: a partial 256-row tile for 129..255 rows left, a 128-row tile below.
    # I = 2048 as in the real layer: one h code that rounds the other way at a boundary (fp32 vs fp64 h)
    # moves a whole y row by ~ulp / sqrt(I), which at I = 256 can reach the 6e-2 element bound.
    "fp8_rest_tiles": get_config("clustered2048_fp8").with_(name="fp8_rest_tiles", routing="random", T=300, H=512,
                                                           E=4, k=2, I=2048, I_shared=2048),
    "fp8_full_and_rest": get_config("decode16_fp8").with_(name="fp8_full_and_rest", T=700, H=512, E=4, k=2,
                                                         I=2048, I_shared=2048),
    # more than 4096 pairs: the three-kernel dispatch, whose scan builds moe_forward's plan
    "many_pairs_fp8": get_config("clustered2048_fp8").with_(name="many_pairs_fp8", routing="zipf", T=1100, H=512,
                                                           E=32, k=4, I=1024, I_shared=1024),
    "many_pairs_bf16": get_config("decode16").with_(name="many_pairs_bf16", routing="random", T=1100, H=512,
                                                   E=64, k=4, I=256, I_shared=256),
    # fp8 with a few rows per expert on average (P / E = 6) but skewed routing: the groups above 32
    # rows take tiles that write fp32 h, quantised with every other row by one launch
    "fp8_few_rows_skewed": get_config("clustered2048_fp8").with_(name="fp8_few_rows_skewed", routing="zipf", T=100,
                                                                H=512, E=64, k=4, I=256, I_shared=256),
    # 512+ bf16 tokens: the LDS-staged router with K split in two, tiled and streaming groups
    "t600_e32_bf16": get_config("decode16").with_(name="t600_e32_bf16", routing="zipf", T=600, H=2048, E=32, k=4,
                                                  I=256, I_shared=256),
    # K / 128 not a multiple of 4 in either GEMM (5 and 9 scale blocks): scales fetched one slice at a time
    "fp8_k_not_4x": get_config("clustered2048_fp8").with_(name="fp8_k_not_4x", routing="random", T=300, H=640,
                                                         E=4, k=2, I=1152, I_shared=1152),
}


def _random_configs(n, seed=2024):
    """n layers drawn from a seeded generator across the accepted shapes:
    1..300 tokens, H and I of several multiples of 64 (of 128 for fp8, with
    I >= 1024 there, where one h code rounding the other way stays within the
    fp8 bound), 1..64 experts, k up to 8, with or without a shared expert,
    random or Zipf routing, and all three weight dtypes (fp8 in both scale
    layouts).  Every draw takes whichever streaming / tiled paths its group
    sizes call for."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kind = ["bf16", "fp8", "fp8_tiles", "f32"][i % 4]
        base = {"bf16": "decode16", "fp8": "clustered2048_fp8", "fp8_tiles": "decode16_fp8", "f32": "tiny_f32"}[kind]
        fp8 = kind.startswith("fp8")
        E = int(rng.integers(1, 65))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.choice([int(rng.integers(1, 33)), int(rng.integers(33, 301))]))
        H = int(rng.choice([256, 384, 512, 768, 1024])) if not fp8 else int(rng.choice([256, 512, 768, 1024]))
        I = int(rng.choice([128, 192, 256, 384, 512])) if not fp8 else int(rng.choice([1024, 1152, 2048]))
        out.append(get_config(base).with_(name=f"rand{i}_{kind}", routing=str(rng.choice(["random", "zipf"])),
                                          T=T, H=H, E=E, k=k, I=I, I_shared=int(rng.choice([0, I]))))
    return out


RANDOM_LAYERS = _random_configs(24)


def _small_inputs(cfg):
    inp = make_inputs(cfg, "cpu")
    gpu = make_inputs(cfg, "cpu")
    for f in ("x", "wg", "bias", "w13", "w2", "ws13", "ws2", "w13_scale", "w2_scale", "ws13_scale", "ws2_scale"):
        t = getattr(gpu, f)
        if t is not None:
            setattr(gpu, f, t.to(DEV))
    return inp, gpu


# ------------------------------------------------------------------ quantiser

@pytest.mark.parametrize("block", [64, 128, 192, 256])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_fp8_bit_exact(dtype, block):
    # 37 rows of 1536: a ragged last workgroup for every block width (the
    # 64/128/256 kernel puts block / 8 lanes on a block, 192 one wave)
    g = torch.Generator().manual_seed(5)
    a = torch.randn(37, 1536, generator=g) * torch.logspace(-6, 3, 1536)[None, :]
    a[3, :768] = 0.0           # all-zero blocks: scale 1
    a[4, :256] = 1e-30         # blocks of subnormal ratios
    a[5, 7] = 448.0 * 3        # saturating neighbourhood of the block maximum
    a = a.to(dtype)
    codes, scales = moe.moe_quantize_fp8(a.to(DEV), block)
    torch.cuda.synchronize()
    oc, os_, _ = oracle.quantize_rows_fp8(oracle.to_f64(a), block)
    np.testing.assert_array_equal(to_np(codes), oc)
    np.testing.assert_array_equal(to_np(scales).astype(np.float64), os_)


# ------------------------------------------------------------------ router

def _route_check(cfg, x, wg, bias):
    mc = moe.cfg_from(cfg)
    idx, w = moe.moe_route(mc, x.to(DEV), wg.to(DEV), bias.to(DEV))
    torch.cuda.synchronize()
    r = oracle.route(oracle.to_f64(x), oracle.to_f64(wg), oracle.to_f64(bias), cfg.k, cfg.score,
                     n_group=cfg.n_group, topk_group=cfg.topk_group)
    near, mism = compare_routing(idx, w, r, cfg.k)
    _log(f"[route {cfg.name}] T={cfg.T} near-ties={near} differing near-tie tokens={len(mism)}")
    return idx, w, r


@pytest.mark.parametrize("name", sorted(SMALL))
def test_route_small(name):
    cfg = SMALL[name]
    x, wg, bias = make_router_inputs(cfg, "cpu")
    _route_check(cfg, x, wg, bias)


@pytest.mark.parametrize("name", ["decode16", "decode256", "prefill8192_ep8", "clustered2048_fp8"])
def test_route_full_size(name):
    cfg = get_config(name)
    x, wg, bias = make_router_inputs(cfg, DEV)
    _route_check(cfg, x.cpu(), wg.cpu(), bias.cpu())


# 512 tokens and more (bf16): the LDS-staged router, one case per expert-count
# class (32, 64, 128, 256 LDS expert rows), with K split over workgroups
# (partial logits + reduce) or in one range (selection in the workgroup),
# ragged token tiles and expert counts below the class size.
_D16, _PF = get_config("decode16"), get_config("prefill8192_ep8")
MANY = {
    "many_e256_split": _D16.with_(name="many_e256_split", T=600, H=2048),
    "many_e256_one_range": _D16.with_(name="many_e256_one_range", T=16400, H=256),
    "many_e200_k6_split": _D16.with_(name="many_e200_k6_split", T=530, H=1024, E=200, k=6),
    "many_e128_split": _D16.with_(name="many_e128_split", T=520, H=2048, E=128),
    "many_e64_split": _D16.with_(name="many_e64_split", T=777, H=4096, E=64),
    "many_e48_softmax_one_range": _D16.with_(name="many_e48_softmax_one_range", T=2100, H=512, E=48, k=4,
                                             score="softmax"),
    "many_e32_split": _PF.with_(name="many_e32_split", T=1000, H=2048),
    "many_e32_one_range": _PF.with_(name="many_e32_one_range", T=700, H=512),
    # K = 384: 6 slices of 64 (not a power of two), exactly 512 tokens (the threshold)
    "many_e64_h384_t512": _D16.with_(name="many_e64_h384_t512", T=512, H=384, E=64, k=6),
    "many_e256_groups_split": _D16.with_(name="many_e256_groups_split", T=1030, H=1024, n_group=8, topk_group=4),
    # fp32 beyond the one-launch router's 64 token tiles: the 16-token split-K
    # kernel with the reduce (69 tiles) and, from 256 tiles, in one K range
    "many_f32_split_reduce": get_config("tiny_f32").with_(name="many_f32_split_reduce", T=1100, H=512),
    "many_f32_one_range": get_config("tiny_f32").with_(name="many_f32_one_range", T=4200, H=256, E=64, k=6),
}


@pytest.mark.parametrize("name", sorted(MANY))
def test_route_many_tokens(name):
    cfg = MANY[name]
    x, wg, bias = make_router_inputs(cfg, "cpu")
    _route_check(cfg, x, wg, bias)


def _random_router_cfgs(n, seed=31):
    """Router shapes on every kernel's side of its limits: 1..3000 tokens
    (the one-launch router below 512 bf16 / 1024 fp32 tokens, the LDS-staged
    or 16-token kernels above), E up to 256 (with expert groups when E has a
    divisor that allows them), k up to 8, sigmoid or softmax, H from 256 to
    4096."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        f32 = i % 3 == 2
        E = int(rng.integers(2, 257))
        k = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(1, 512)) if i % 2 == 0 else int(rng.integers(512, 3001))
        H = 128 * int(rng.integers(2, 33))
        score = str(rng.choice(["sigmoid", "softmax"]))
        ng = [g for g in (2, 4, 8) if E % g == 0 and E // g >= 2 and k <= (E // g) * max(1, g // 2)]
        n_group = int(rng.choice(ng)) if ng and rng.random() < 0.4 else 1
        topk_group = max(1, n_group // 2)
        base = get_config("tiny_f32") if f32 else get_config("decode16")
        out.append(base.with_(name=f"route_rand{i}", routing=str(rng.choice(["random", "zipf"])), T=T, H=H, E=E,
                              k=k, score=score, n_group=n_group, topk_group=topk_group))
    return out


ROUTER_RANDOM = _random_router_cfgs(18)


@pytest.mark.parametrize("cfg", ROUTER_RANDOM, ids=[c.name for c in ROUTER_RANDOM])
def test_route_random_shapes(cfg):
    _log(f"[route random] {cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} {cfg.score} {cfg.act_dtype} "
         f"groups {cfg.n_group}/{cfg.topk_group}")
    x, wg, bias = make_router_inputs(cfg, "cpu")
    _route_check(cfg, x, wg, bias)


@pytest.mark.parametrize("name", ["decode16", "decode256"])
def test_route_one_launch_leaves_counters_zero(name):
    """The one-launch router counts finished workgroups per token tile in the
    workspace's first 256 bytes: after each call they are zero again, and a
    second call on the same workspace gives the same bits."""
    cfg = get_config(name)
    x, wg, bias = make_router_inputs(cfg, DEV)
    mc = moe.cfg_from(cfg)
    ws = moe.alloc_workspace(mc)
    idx1, w1 = moe.moe_route(mc, x, wg, bias, ws=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:256]) == 0
    idx2, w2 = moe.moe_route(mc, x, wg, bias, ws=ws)
    torch.cuda.synchronize()
    assert torch.count_nonzero(ws[:256]) == 0
    assert torch.equal(idx1, idx2) and torch.equal(w1, w2)


# Group-limited routing: DeepSeek-V3-like groups (256 experts in 8 groups,
# 4 kept) on the split-K router, a prefill-sized call on the LDS-staged
# router, softmax scoring in fp32, and the all-groups case.
GROUPED = {
    "groups_e256_g8_t4": get_config("decode16").with_(name="groups_e256_g8_t4", T=64, H=1024, n_group=8,
                                                     topk_group=4),
    "groups_e32_g4_t2_fused": get_config("prefill8192_ep8").with_(name="groups_e32_g4_t2_fused", n_group=4,
                                                                  topk_group=2),
    "groups_e16_g4_t2_f32": get_config("tiny_f32").with_(name="groups_e16_g4_t2_f32", T=37, n_group=4,
                                                          topk_group=2, k=3),
    "groups_all_e64": get_config("decode16").with_(name="groups_all_e64", T=40, H=512, E=64, n_group=8,
                                                   topk_group=8),
}


@pytest.mark.parametrize("name", sorted(GROUPED))
def test_route_group_limited(name):
    cfg = GROUPED[name]
    x, wg, bias = make_router_inputs(cfg, "cpu")
    idx, _, r = _route_check(cfg, x, wg, bias)
    gs = cfg.E // cfg.n_group
    groups = to_np(idx).astype(np.int64) // gs
    assert max(len(set(row.tolist())) for row in groups) <= cfg.topk_group
    if cfg.topk_group < cfg.n_group:
        plain = oracle.route(oracle.to_f64(x), oracle.to_f64(wg), oracle.to_f64(bias), cfg.k, cfg.score)
        assert (plain["idx"] != r["idx"]).any(), "the group stage changed nothing: a weak test case"


def test_forward_group_limited():
    cfg = get_config("decode16").with_(name="forward_groups", T=48, H=512, E=32, k=4, I=256, I_shared=256,
                                       n_group=8, topk_group=2)
    inp, gin = _small_inputs(cfg)
    ref = oracle.forward(inp)
    y, idx, w, counts = moe.moe_forward(moe.cfg_from(cfg), gin.x, gin.wg, gin.bias, moe.Weights.from_inputs(gin),
                                        return_routing=True)
    torch.cuda.synchronize()
    _, mism = compare_routing(idx, w, ref["route"], cfg.k)
    keep = np.setdiff1d(np.arange(cfg.T), mism)
    assert_outputs_close(to_np(y)[keep], ref["y"][keep], tol_key(cfg), "y")


# ------------------------------------------------------------------ routing statistics

@pytest.mark.parametrize("name,n_ranks", [("decode16", 8), ("decode256", 8), ("prefill8192_ep8", 4),
                                          ("clustered2048_fp8", 16), ("tiny_f32", 1)])
def test_routing_stats_exact(name, n_ranks):
    """Loads, skews and the affinity matrix of the oracle's own routing of
    each workload (the input is the oracle's top-k, so GPU routing near ties
    do not enter): integers bit-exact, skews to fp32 rounding."""
    cfg = get_config(name)
    x, wg, bias = make_router_inputs(cfg, "cpu")
    r = oracle.route(oracle.to_f64(x), oracle.to_f64(wg), oracle.to_f64(bias), cfg.k, cfg.score)
    ref = oracle.routing_stats(r["idx"], cfg.E, n_ranks)
    idx = torch.from_numpy(r["idx"].astype(np.int32)).to(DEV)
    counts, rank_load, skew, aff = moe.moe_routing_stats(moe.cfg_from(cfg), idx, n_ranks)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(counts), ref["counts"])
    np.testing.assert_array_equal(to_np(rank_load), ref["rank_load"])
    np.testing.assert_array_equal(to_np(aff), ref["affinity"])
    np.testing.assert_allclose(to_np(skew), [ref["rho_rank"], ref["rho_expert"]], rtol=2e-7)
    _log(f"[stats {name}] rho over {n_ranks} ranks {ref['rho_rank']:.3f}, over experts {ref['rho_expert']:.3f}")


def test_routing_stats_skips_out_of_range_and_optional_outputs():
    cfg = get_config("tiny_f32").with_(T=5, k=2, E=16)
    idx = torch.tensor([[0, 1], [2, 3], [-1, 4], [16, 5], [6, 7]], dtype=torch.int32, device=DEV)
    counts, rank_load, skew, aff = moe.moe_routing_stats(moe.cfg_from(cfg), idx, 2, affinity=False)
    torch.cuda.synchronize()
    assert aff is None
    expect = np.zeros(16, dtype=np.int64)
    expect[:8] = 1                       # -1 and 16 are skipped
    np.testing.assert_array_equal(to_np(counts), expect)
    np.testing.assert_array_equal(to_np(rank_load), [8, 0])


# ------------------------------------------------------------------ dispatch

def _distinct_topk(rng, T, E, k):
    return np.argsort(rng.random((T, E)), axis=1)[:, :k]


# single-workgroup path up to 4096 pairs (several 1024-pair chunks at 512 x 8),
# the three-kernel path above (513 x 8 = 4104 pairs and more)
@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (33, 4, 4), (200, 32, 4), (1000, 256, 8), (8192, 32, 8),
                                   (2048, 256, 8), (16, 256, 8), (512, 256, 8), (513, 256, 8), (300, 3, 2)])
def test_dispatch_exact(T, E, k):
    rng = np.random.default_rng(T * 7 + E)
    idx = _distinct_topk(rng, T, E, k)
    cfg = moe.make_cfg(T, 128, E, k, 64, 64)
    got = moe.moe_dispatch(cfg, torch.from_numpy(idx.astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx, E)
    for name, g in zip(("counts", "offsets", "sorted_pair", "pair_slot"), got):
        np.testing.assert_array_equal(to_np(g), ref[name], err_msg=name)


def _random_dispatch_shapes(n, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        E = int(rng.integers(1, 257))
        k = int(rng.integers(1, min(E, 32) + 1))
        T = int(rng.integers(1, 20000 // k + 2))
        out.append((T, E, k, bool(rng.random() < 0.5)))
    return out


@pytest.mark.parametrize("T,E,k,skew", _random_dispatch_shapes(16))
def test_dispatch_random_shapes(T, E, k, skew):
    """Seeded random shapes on both sides of the one-workgroup limit (4096
    pairs), with uniform or skewed expert choice (a few experts taking most
    pairs), bit-exact against the oracle's dispatch."""
    rng = np.random.default_rng(T * 131 + E * 7 + k)
    if skew:   # distinct experts per token, drawn with Zipf-like weights
        p = 1.0 / np.arange(1, E + 1) ** 1.2
        idx = np.stack([rng.choice(E, size=k, replace=False, p=p / p.sum()) for _ in range(T)])
    else:
        idx = _distinct_topk(rng, T, E, k)
    cfg = moe.make_cfg(T, 128, E, k, 64, 64)
    got = moe.moe_dispatch(cfg, torch.from_numpy(idx.astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx, E)
    for name, g in zip(("counts", "offsets", "sorted_pair", "pair_slot"), got):
        np.testing.assert_array_equal(to_np(g), ref[name], err_msg=name)


def test_dispatch_maximum_pairs():
    """The largest call the library accepts, T * k = 2^24 pairs (E = 256,
    k = 8), against the definitions the oracle's loops are pinned to (too
    slow for its plain loops here): counts = bincount, offsets = exclusive
    cumsum, sorted_pair = stable argsort of the expert ids, pair_slot = its
    inverse."""
    T, E, k = 1 << 21, 256, 8
    rng = np.random.default_rng(24)
    base = rng.integers(0, E, size=(T, 1))
    step = 2 * rng.integers(0, E // 2, size=(T, 1)) + 1          # odd: k distinct experts per token
    idx = ((base + step * np.arange(k)[None, :]) % E).astype(np.int32)
    cfg = moe.make_cfg(T, 128, E, k, 64, 64)
    got = moe.moe_dispatch(cfg, torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    sorted_pair = np.argsort(flat, kind="stable")
    pair_slot = np.empty_like(sorted_pair)
    pair_slot[sorted_pair] = np.arange(flat.shape[0])
    for name, g, r in zip(("counts", "offsets", "sorted_pair", "pair_slot"), got,
                          (counts, offsets, sorted_pair, pair_slot)):
        np.testing.assert_array_equal(to_np(g), r, err_msg=name)


@pytest.mark.parametrize("T,E,k", [(40, 16, 4), (1200, 32, 8)])
def test_dispatch_and_combine_skip_out_of_range_ids(T, E, k):
    """Ids outside [0, E) are the library's documented invalid input: the
    dispatch counts them nowhere and gives their pairs pair_slot = -1, and
    the combine adds nothing for them.  Both the one-workgroup dispatch
    (160 pairs) and the three-kernel one (9600 pairs) are covered; the
    expected values are the definitions restricted to the valid pairs."""
    rng = np.random.default_rng(T + E)
    idx = _distinct_topk(rng, T, E, k).astype(np.int64)
    bad = rng.random(idx.shape) < 0.1
    idx[bad] = rng.choice([-1, -7, E, E + 3], size=int(bad.sum()))
    cfg = moe.make_cfg(T, 128, E, k, 64, 64)
    counts, offsets, sorted_pair, pair_slot = moe.moe_dispatch(cfg, torch.from_numpy(idx.astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    ref_counts = np.bincount(flat[valid], minlength=E)
    ref_off = np.concatenate([[0], np.cumsum(ref_counts)])
    ref_sorted = np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")]
    ref_slot = np.full(flat.shape[0], -1)
    ref_slot[ref_sorted] = np.arange(len(ref_sorted))
    np.testing.assert_array_equal(to_np(counts), ref_counts)
    np.testing.assert_array_equal(to_np(offsets), ref_off)
    np.testing.assert_array_equal(to_np(sorted_pair)[:len(ref_sorted)], ref_sorted)
    np.testing.assert_array_equal(to_np(pair_slot), ref_slot)
    # combine: rows of y_sorted in bf16, weights in fp32; skipped pairs add nothing
    H = 128
    ys = torch.from_numpy(rng.standard_normal((T * k, H))).to(torch.bfloat16)
    ysh = torch.from_numpy(rng.standard_normal((T, H))).to(torch.bfloat16)
    w = torch.from_numpy(rng.random((T, k)).astype(np.float32))
    y = moe.moe_combine(cfg, ys.to(DEV), ysh.to(DEV), pair_slot, w.to(DEV))
    torch.cuda.synchronize()
    ys64, w64 = oracle.to_f64(ys), w.double().numpy()
    expect = oracle.to_f64(ysh).copy()
    for t in range(T):
        for j in range(k):
            if valid[t * k + j]:
                expect[t] += w64[t, j] * ys64[ref_slot[t * k + j]]
    assert_outputs_close(y, expect, "bf16", "combine with skipped pairs")


@pytest.mark.parametrize("T", [4096, 65536])
def test_dispatch_all_pairs_to_one_expert(T):
    E, k = 8, 1
    idx = np.full((T, k), 5)
    cfg = moe.make_cfg(T, 128, E, k, 64, 64)
    got = moe.moe_dispatch(cfg, torch.from_numpy(idx.astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.dispatch(idx, E)
    for name, g in zip(("counts", "offsets", "sorted_pair", "pair_slot"), got):
        np.testing.assert_array_equal(to_np(g), ref[name], err_msg=name)


# ------------------------------------------------------------------ expert FFN and combine (stage by stage)

@pytest.mark.parametrize("name", sorted(SMALL))
def test_expert_ffn_small(name):
    cfg = SMALL[name]
    inp, gin = _small_inputs(cfg)
    ref = oracle.forward(inp)
    d = ref["dispatch"]
    mc = moe.cfg_from(cfg)
    off = torch.from_numpy(d["offsets"].astype(np.int32)).to(DEV)
    sp = torch.from_numpy(d["sorted_pair"].astype(np.int32)).to(DEV)
    ys, ysh = moe.moe_expert_ffn(mc, gin.x, off, sp, moe.Weights.from_inputs(gin))
    torch.cuda.synchronize()
    key = tol_key(cfg)
    e1 = assert_outputs_close(ys, ref["y_sorted"], key, "y_sorted")
    if cfg.I_shared:
        e2 = assert_outputs_close(ysh, ref["y_shared"], key, "y_shared")
    else:
        e2 = None
    _log(f"[expert_ffn {name}] y_sorted err {e1} y_shared err {e2}")


@pytest.mark.parametrize("sizes", [[129] * 4, [385, 129, 129, 129], [385, 129, 33, 5, 0]])
def test_expert_ffn_fp8_tile_bound(sizes):
    """Crafted group sizes at the 256-row tile grid's bound.  With 128-row rest
    tiles (fp8) every 256-row tile, full or partial, holds at least 129 rows,
    so a launch of P // 129 tiles covers them all; groups of 129 and 256 + 129
    rows reach that bound exactly.  The last case adds a 128-row rest tile, a
    streaming group and an empty group."""
    E, T = len(sizes), sum(sizes)
    cfg = get_config("clustered2048_fp8").with_(name="fp8_tile_bound", routing="random", T=T, H=512, E=E, k=1,
                                                I=2048, I_shared=0)
    inp, gin = _small_inputs(cfg)
    # k = 1: pair p is token p; any order within a group is a valid dispatch
    sorted_pair = np.random.default_rng(5).permutation(T).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    ow = oracle.OracleWeights.from_inputs(inp)
    xa = oracle.prepare_activations(inp.x.double().numpy(), ow.fp8, ow.block)
    ref_ys, _ = oracle.expert_ffn(xa, offsets, sorted_pair, 1, ow)
    ys, _ = moe.moe_expert_ffn(moe.cfg_from(cfg), gin.x, torch.from_numpy(offsets).to(DEV),
                               torch.from_numpy(sorted_pair).to(DEV), moe.Weights.from_inputs(gin))
    torch.cuda.synchronize()
    e = assert_outputs_close(ys, ref_ys, tol_key(cfg), "y_sorted")
    _log(f"[expert_ffn tile bound {sizes}] y_sorted err {e}")


BOUNDARY_SIZES = [1, 8, 9, 16, 17, 32, 33, 64, 127, 128, 129, 255, 256, 257, 511, 513, 0]


@pytest.mark.parametrize("kind", ["bf16", "f32", "fp8", "fp8_tiles"])
def test_expert_ffn_group_size_boundaries(kind):
    """One group at every row-count boundary of the work lists (the 8 / 16 /
    32-row streaming classes, 128-row rest tiles, 256-row tiles and their
    partial tails) and an empty group, k = 1, with a shared expert of all
    their rows, in each weight dtype."""
    sizes = BOUNDARY_SIZES
    E, T = len(sizes), sum(sizes)
    base = {"bf16": "decode16", "f32": "tiny_f32", "fp8": "clustered2048_fp8", "fp8_tiles": "decode16_fp8"}[kind]
    I = 2048 if kind.startswith("fp8") else 256
    cfg = get_config(base).with_(name=f"boundaries_{kind}", routing="random", T=T, H=512, E=E, k=1, I=I, I_shared=I)
    _log(f"[expert_ffn boundaries {kind}] T={T} E={E}")
    inp, gin = _small_inputs(cfg)
    sorted_pair = np.random.default_rng(11).permutation(T).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    ow = oracle.OracleWeights.from_inputs(inp)
    xa = oracle.prepare_activations(inp.x.double().numpy(), ow.fp8, ow.block)
    ref_ys, ref_sh = oracle.expert_ffn(xa, offsets, sorted_pair, 1, ow)
    ys, ysh = moe.moe_expert_ffn(moe.cfg_from(cfg), gin.x, torch.from_numpy(offsets).to(DEV),
                                 torch.from_numpy(sorted_pair).to(DEV), moe.Weights.from_inputs(gin))
    torch.cuda.synchronize()
    e = assert_outputs_close(ys, ref_ys, tol_key(cfg), "y_sorted")
    e2 = assert_outputs_close(ysh, ref_sh, tol_key(cfg), "y_shared")
    _log(f"[expert_ffn boundaries {kind}] y_sorted err {e} y_shared err {e2}")


@pytest.mark.parametrize("sizes,shared", [([255, 240, 208, 193, 192, 176, 145, 130, 511], False),
                                          ([300, 150, 40, 7], True)])
def test_expert_ffn_fp8_partial_tiles(sizes, shared):
    """fp8 256-row tiles give wave wm the 16-row M tiles wm, wm + 4, ... and
    skip the activation loads of 8-row blocks past a partial tile's rows:
    rests of 130..255 rows (and 511 = 256 + 255) put the last valid M tile
    at every wave in turn.  The second case has a shared expert of 497
    tokens: one full 256-row tile (fp8 GEMM1 on 128-column tiles) and two
    128-row tiles for the rest, beside a partial 256-row routed tile."""
    E, T = len(sizes), sum(sizes)
    cfg = get_config("clustered2048_fp8").with_(name="fp8_partial_tiles", routing="random", T=T, H=512, E=E, k=1,
                                                I=2048, I_shared=2048 if shared else 0)
    inp, gin = _small_inputs(cfg)
    sorted_pair = np.random.default_rng(7).permutation(T).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    ow = oracle.OracleWeights.from_inputs(inp)
    xa = oracle.prepare_activations(inp.x.double().numpy(), ow.fp8, ow.block)
    ref_ys, ref_sh = oracle.expert_ffn(xa, offsets, sorted_pair, 1, ow)
    ys, ysh = moe.moe_expert_ffn(moe.cfg_from(cfg), gin.x, torch.from_numpy(offsets).to(DEV),
                                 torch.from_numpy(sorted_pair).to(DEV), moe.Weights.from_inputs(gin))
    torch.cuda.synchronize()
    e = assert_outputs_close(ys, ref_ys, tol_key(cfg), "y_sorted")
    e2 = assert_outputs_close(ysh, ref_sh, tol_key(cfg), "y_shared") if shared else None
    _log(f"[expert_ffn fp8 partial tiles {sizes}] y_sorted err {e} y_shared err {e2}")


# The expert FFN's two GEMMs one at a time.  GEMM1 + SwiGLU: the h that
# moe_expert_ffn leaves in the workspace (moe_workspace_ffn_h) against the
# oracle's h, and for fp8 its codes and scales against the oracle's h within
# the rounding of E4M3.  GEMM2: the oracle's h (its bf16 or fp32 rounding, or
# for fp8 the oracle's codes and scales of it) written into a fresh workspace,
# then moe_expert_ffn_down, against the oracle's product of that same h with
# W2.  Fed the same h, GEMM2 must agree to the output's own rounding, also at
# I = 256, where in the whole layer one h code rounding the other way (fp32
# vs fp64 h) moves a y row visibly.
FFN_STAGES = ["small_fp8", "t12_fp8", "t20_fp8", "small_fp8_tiles", "fp8_k_not_4x", "fp8_rest_tiles",
              "fp8_few_rows_skewed", "small_bf16",
              "t16_e4_halves_bf16", "t24_bf16", "t600_e32_bf16", "k_eq_E_bf16", "tiny_f32", "t20_f32"]

# GEMM2 on a given h: fp32 accumulation, then one rounding to the output
# type.  bf16 keeps 8 significant bits, so that rounding moves an element by
# at most 2^-8 of its value: per element (relative to max(|o|, rms(o)))
# 2^-8 plus 1/16 of it for the fp32 sums, and 2^-8 in Frobenius norm.  fp32
# outputs stay within the fp32 bounds.
GEMM2_TOL = {"bf16": (2.0 ** -8 * 1.0625, 2.0 ** -8), "f32": (1e-4, 1e-5)}


def _h_fp32_bound(a, w1, w3):
    """Per-element bound on an fp32 h = SiLU(g) * u, g = a W1^T, u = a W3^T,
    against exact arithmetic: a K-term fp32 sum in any order is within
    K 2^-24 of the sum of its terms' magnitudes (plus one rounding per scale
    multiply, hence K + 2), and the error of g and u reaches h through
    |SiLU'(g)| |u| and |SiLU(g)|; SiLU's own roundings add a few ulps of h."""
    g, u = a @ w1.T, a @ w3.T
    ga, ua = np.abs(a) @ np.abs(w1).T, np.abs(a) @ np.abs(w3).T
    s = 1.0 / (1.0 + np.exp(-g))
    dsilu = s * (1.0 + g * (1.0 - s))
    gamma = (a.shape[1] + 2) * 2.0 ** -24
    return gamma * (np.abs(dsilu) * ga * np.abs(u) + np.abs(g * s) * ua) + 2.0 ** -20 * np.abs(g * s * u)


def _ws_view(ws, off, rows, cols, dtype):
    n = rows * cols * torch.empty((), dtype=dtype).element_size()
    return ws[off:off + n].view(dtype).reshape(rows, cols)


def _ffn_stage_cases():
    return [SMALL[n] for n in FFN_STAGES] + RANDOM_LAYERS[::3]


@pytest.mark.parametrize("cfg", _ffn_stage_cases(), ids=[c.name for c in _ffn_stage_cases()])
def test_expert_ffn_gemm1_and_gemm2_apart(cfg):
    name = cfg.name
    inp, gin = _small_inputs(cfg)
    ow = oracle.OracleWeights.from_inputs(inp)
    x = oracle.to_f64(inp.x)
    r = oracle.route(x, oracle.to_f64(inp.wg), oracle.to_f64(inp.bias), cfg.k, cfg.score,
                     n_group=cfg.n_group, topk_group=cfg.topk_group)
    d = oracle.dispatch(r["idx"], cfg.E)
    xa = oracle.prepare_activations(x, ow.fp8, ow.block)
    T, k, I, P, qb = cfg.T, cfg.k, cfg.I, cfg.T * cfg.k, cfg.quant_block
    rows = P + (T if cfg.I_shared else 0)

    # (rows of h, tokens, weights) per routed group, then the shared expert
    parts = []
    for e in range(cfg.E):
        lo, hi = int(d["offsets"][e]), int(d["offsets"][e + 1])
        if hi > lo:
            parts.append((slice(lo, hi), np.asarray(d["sorted_pair"][lo:hi]) // k, ow.expert(e)))
    if cfg.I_shared:
        parts.append((slice(P, P + T), np.arange(T), ow.shared()))
    used = np.zeros(rows, dtype=bool)
    h_ref = np.zeros((rows, I))
    h_bound = np.zeros((rows, I))
    for sl, toks, (w1, w3, _) in parts:
        used[sl] = True
        h_ref[sl] = oracle.swiglu_hidden(xa[toks], w1, w3)
        h_bound[sl] = _h_fp32_bound(xa[toks], w1, w3)

    mc = moe.cfg_from(cfg)
    wts = moe.Weights.from_inputs(gin)
    off = torch.from_numpy(d["offsets"].astype(np.int32)).to(DEV)
    sp = torch.from_numpy(d["sorted_pair"].astype(np.int32)).to(DEV)
    h_off, hq_off, hs_off = moe.moe_workspace_ffn_h(mc)
    h_dt = torch.bfloat16 if cfg.w_dtype == "bf16" else torch.float32

    # GEMM1 + SwiGLU (and for fp8 the quantisation of h)
    ws = moe.alloc_workspace(mc, DEV)
    ys_full, ysh_full = moe.moe_expert_ffn(mc, gin.x, off, sp, wts, ws=ws)
    # the down projection alone on the h that call left runs the same kernels: the same bits
    ys_down, ysh_down = moe.moe_expert_ffn_down(mc, off, sp, wts, ws)
    torch.cuda.synchronize()
    valid = int(d["offsets"][-1])
    assert torch.equal(ys_down[:valid], ys_full[:valid])
    if cfg.I_shared:
        assert torch.equal(ysh_down, ysh_full)
    h_gpu = to_np(_ws_view(ws, h_off, rows, I, h_dt))[used]
    if cfg.w_dtype == "bf16":   # h rounded once to bf16
        eh = assert_outputs_close(h_gpu, h_ref[used], "bf16", "h")
    elif cfg.w_dtype == "f32":
        ratio = np.abs(h_gpu - h_ref[used]) / np.maximum(h_bound[used], 1e-300)
        eh = (float(ratio.max()), output_errors(h_gpu, h_ref[used]))
        assert eh[0] <= 1.0, f"h beyond its fp32 accumulation bound: worst error / bound {eh[0]:.3e}, {eh[1]}"
    else:   # fp8: the codes and scales below are the output (tiled groups never write h itself)
        eh = None
    if ow.fp8:
        # E4M3 keeps 4 significant bits (rounding within 2^-4 of a normal
        # value) and steps by 2^-9 below 2^-6, in units of the block scale
        codes = to_np(_ws_view(ws, hq_off, rows, I, torch.uint8))[used]
        scales = to_np(_ws_view(ws, hs_off, rows, I // qb, torch.float32))[used]
        deq = oracle.e4m3_decode(codes) * np.repeat(scales, qb, axis=1)
        ref_scale = np.repeat(oracle.quantize_rows_fp8(h_ref[used], qb)[1], qb, axis=1)
        qbound = 2.0 ** -4 * np.abs(h_ref[used]) + 1.07 * h_bound[used] + 2.0 ** -10 * 1.01 * ref_scale
        qr = float((np.abs(deq - h_ref[used]) / qbound).max())
        assert qr <= 1.0, f"h codes and scales beyond E4M3 rounding of h: worst error / bound {qr:.3e}"
        # the scales themselves: amax / 448 of h, within h's fp32 error
        ref_s = oracle.quantize_rows_fp8(h_ref[used], qb)[1]
        amax_bound = np.max((h_bound[used]).reshape(-1, I // qb, qb), axis=2) / 448.0
        assert np.all(np.abs(scales - ref_s) <= 1.01 * amax_bound + 2.0 ** -23 * ref_s), "h scales"
        eh = ("codes / E4M3 bound", qr)

    # GEMM2 alone on the oracle's h
    ws2 = moe.alloc_workspace(mc, DEV)
    y_ref = np.zeros((rows, cfg.H))
    if ow.fp8:
        codes, scales, h_in = oracle.quantize_rows_fp8(h_ref, qb)
        _ws_view(ws2, hq_off, rows, I, torch.uint8).copy_(torch.from_numpy(codes))
        _ws_view(ws2, hs_off, rows, I // qb, torch.float32).copy_(torch.from_numpy(scales.astype(np.float32)))
    else:
        h_t = torch.from_numpy(h_ref).to(h_dt)
        _ws_view(ws2, h_off, rows, I, h_dt).copy_(h_t)
        h_in = h_t.double().numpy()
    for sl, _, (_, _, w2) in parts:
        y_ref[sl] = h_in[sl] @ w2.T
    ys, ysh = moe.moe_expert_ffn_down(mc, off, sp, wts, ws2)
    torch.cuda.synchronize()
    y_gpu = to_np(ys) if not cfg.I_shared else np.concatenate([to_np(ys), to_np(ysh)])
    el, fr = output_errors(y_gpu[used], y_ref[used])
    tol = GEMM2_TOL[cfg.act_dtype]
    assert el <= tol[0] and fr <= tol[1], f"GEMM2 on the oracle's h: elementwise {el:.3e}, Frobenius {fr:.3e}, tol {tol}"
    _log(f"[ffn gemm1/gemm2 {name}] h err {eh} GEMM2 err ({el:.3e}, {fr:.3e})")


@pytest.mark.parametrize("name", sorted(SMALL))
def test_combine_small(name):
    cfg = SMALL[name]
    inp, _ = _small_inputs(cfg)
    ref = oracle.forward(inp)
    # the stage's inputs in the activation dtype, as moe_expert_ffn stores them
    adt = torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16
    ys_in = torch.from_numpy(ref["y_sorted"]).to(adt)
    ysh_in = torch.from_numpy(ref["y_shared"]).to(adt)
    w32 = ref["route"]["w"].astype(np.float32)
    expect = oracle.combine(oracle.to_f64(ys_in), oracle.to_f64(ysh_in) if cfg.I_shared else np.zeros_like(ref["y_shared"]),
                            ref["dispatch"]["pair_slot"], w32.astype(np.float64), cfg.k)
    mc = moe.cfg_from(cfg)
    y = moe.moe_combine(mc, ys_in.to(DEV),
                        ysh_in.to(DEV) if cfg.I_shared else None,
                        torch.from_numpy(ref["dispatch"]["pair_slot"].astype(np.int32)).to(DEV),
                        torch.from_numpy(w32).to(DEV))
    torch.cuda.synchronize()
    key = "f32" if cfg.act_dtype == "f32" else "bf16"
    assert_outputs_close(y, expect, key, "combine")


# ------------------------------------------------------------------ whole layer

@pytest.mark.parametrize("name", sorted(SMALL))
def test_forward_small(name):
    cfg = SMALL[name]
    inp, gin = _small_inputs(cfg)
    ref = oracle.forward(inp)
    mc = moe.cfg_from(cfg)
    y, idx, w, counts = moe.moe_forward(mc, gin.x, gin.wg, gin.bias, moe.Weights.from_inputs(gin),
                                        return_routing=True)
    torch.cuda.synchronize()
    near, mism = compare_routing(idx, w, ref["route"], cfg.k)
    keep = np.setdiff1d(np.arange(cfg.T), mism)
    if len(mism) == 0:
        np.testing.assert_array_equal(to_np(counts), ref["dispatch"]["counts"])
    err = assert_outputs_close(to_np(y)[keep], ref["y"][keep], tol_key(cfg), "y")
    _log(f"[forward {name}] near-ties={near} excluded={len(mism)} err={err}")


@pytest.mark.parametrize("cfg", RANDOM_LAYERS, ids=[c.name for c in RANDOM_LAYERS])
def test_forward_random_layers(cfg):
    _log(f"[forward random] {cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I} "
         f"I_shared={cfg.I_shared} {cfg.w_dtype} {cfg.routing}")
    inp, gin = _small_inputs(cfg)
    ref = oracle.forward(inp)
    y, idx, w, counts = moe.moe_forward(moe.cfg_from(cfg), gin.x, gin.wg, gin.bias, moe.Weights.from_inputs(gin),
                                        return_routing=True)
    torch.cuda.synchronize()
    near, mism = compare_routing(idx, w, ref["route"], cfg.k)
    keep = np.setdiff1d(np.arange(cfg.T), mism)
    err = assert_outputs_close(to_np(y)[keep], ref["y"][keep], tol_key(cfg), "y")
    _log(f"[forward random {cfg.name}] near-ties={near} excluded={len(mism)} err={err}")


@pytest.mark.parametrize("name", ["tiny_f32", "small_bf16", "small_fp8", "t16_e4_halves_bf16", "t600_e32_bf16",
                                  "many_pairs_fp8", "many_pairs_bf16"])
def test_forward_matches_stages_bitwise(name):
    """moe_forward builds the FFN work lists inside its dispatch (up to 4096
    pairs in the one-workgroup kernel, above that in the scan kernel); the
    stage entry points build them in the FFN's own plan kernel.  Both must
    give the same bits (t600_e32_bf16, 2400 pairs, also takes the LDS-staged
    router; the many_pairs layers, 4400 pairs, the three-kernel dispatch)."""
    cfg = SMALL[name]
    _, gin = _small_inputs(cfg)
    mc = moe.cfg_from(cfg)
    wts = moe.Weights.from_inputs(gin)
    y, idx, w, counts = moe.moe_forward(mc, gin.x, gin.wg, gin.bias, wts, return_routing=True)
    idx2, w2 = moe.moe_route(mc, gin.x, gin.wg, gin.bias)
    counts2, off2, sp2, slot2 = moe.moe_dispatch(mc, idx2)
    ys, ysh = moe.moe_expert_ffn(mc, gin.x, off2, sp2, wts)
    y2 = moe.moe_combine(mc, ys, ysh, slot2, w2)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(w, w2) and torch.equal(counts, counts2)
    assert torch.equal(y, y2)


def test_forward_is_deterministic():
    cfg = SMALL["small_bf16"]
    _, gin = _small_inputs(cfg)
    mc = moe.cfg_from(cfg)
    ws = moe.alloc_workspace(mc)
    outs = [moe.moe_forward(mc, gin.x, gin.wg, gin.bias, moe.Weights.from_inputs(gin), ws=ws, return_routing=True)
            for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_forward_on_user_stream_is_ordered():
    """The call forks the shared expert (T > 32) onto a side stream and joins
    it back: work queued after it on the caller's stream sees the whole
    output, without a device-wide synchronisation in between."""
    cfg = SMALL["small_bf16"]
    inp, gin = _small_inputs(cfg)
    ref = oracle.forward(inp)
    mc = moe.cfg_from(cfg)
    ws = moe.alloc_workspace(mc)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        copies = []
        for _ in range(2):
            out = moe.moe_forward(mc, gin.x, gin.wg, gin.bias, moe.Weights.from_inputs(gin), ws=ws,
                                  return_routing=True)
            copies.append([t.clone() for t in out])      # queued on s right after the call
    s.synchronize()
    for y, idx, w, _ in copies:
        _, mism = compare_routing(idx, w, ref["route"], cfg.k)
        keep = np.setdiff1d(np.arange(cfg.T), mism)
        assert_outputs_close(to_np(y)[keep], ref["y"][keep], tol_key(cfg), "y")


GRAPH_CASES = [SMALL[n] for n in ("tiny_f32", "small_bf16", "t24_bf16", "small_fp8", "t600_e32_bf16",
                                   "fp8_k_not_4x")] + RANDOM_LAYERS[2::5]


@pytest.mark.parametrize("cfg", GRAPH_CASES, ids=[c.name for c in GRAPH_CASES])
def test_graph_replays_match_eager(cfg):
    """A captured whole-layer graph, replayed several times with eager work
    and synchronisations in between, gives the eager result bit for bit
    (the layer is deterministic), and follows a change of routing: the
    per-expert counts are read on the device at every launch."""
    inp, gin = _small_inputs(cfg)
    mc = moe.cfg_from(cfg)
    w = moe.Weights.from_inputs(gin)
    y_ref = moe.moe_forward(mc, gin.x, gin.wg, gin.bias, w)
    torch.cuda.synchronize()
    x = gin.x.clone()
    ws = moe.alloc_workspace(mc)
    y = torch.empty_like(y_ref)
    g = moe.MoEGraph(mc, x, gin.wg, gin.bias, w, y, ws)
    for rep in range(3):
        y.zero_()
        g.launch()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}"
        scratch = moe.moe_forward(mc, gin.x, gin.wg, gin.bias, w)     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(scratch, y_ref)
    # new routing: the graph must equal an eager call on the new input
    x.copy_(torch.roll(gin.x, 1, dims=1))
    y_new = moe.moe_forward(mc, x, gin.wg, gin.bias, w)
    g.launch()
    torch.cuda.synchronize()
    assert torch.equal(y, y_new)
    assert not torch.equal(y_new, y_ref)
    g.close()


def test_graph_full_size_decode16():
    cfg = get_config("decode16")
    gin = make_inputs(cfg, DEV)
    mc = moe.cfg_from(cfg)
    w = moe.Weights.from_inputs(gin)
    y_ref = moe.moe_forward(mc, gin.x, gin.wg, gin.bias, w)
    ws = moe.alloc_workspace(mc)
    y = torch.empty_like(y_ref)
    g = moe.MoEGraph(mc, gin.x, gin.wg, gin.bias, w, y, ws)
    for _ in range(3):
        g.launch()
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    g.close()


def test_zero_input_gives_zero_output():
    cfg = SMALL["small_bf16"]
    _, gin = _small_inputs(cfg)
    gin.x.zero_()
    y = moe.moe_forward(moe.cfg_from(cfg), gin.x, gin.wg, gin.bias, moe.Weights.from_inputs(gin))
    torch.cuda.synchronize()
    assert torch.count_nonzero(y) == 0


def test_all_tokens_to_one_expert():
    """A +10 selection bias on one expert sends every token there (k = 1): one
    group with all T rows takes the tiled regime with a ragged last tile."""
    cfg = SMALL["small_bf16"].with_(name="hot_expert", T=300, k=1)
    inp, gin = _small_inputs(cfg)
    inp.bias[7] = 10.0
    gin.bias[7] = 10.0
    ref = oracle.forward(inp)
    assert (ref["route"]["idx"] == 7).all()
    y, idx, w, counts = moe.moe_forward(moe.cfg_from(cfg), gin.x, gin.wg, gin.bias, moe.Weights.from_inputs(gin),
                                        return_routing=True)
    torch.cuda.synchronize()
    assert (to_np(idx) == 7).all()
    np.testing.assert_array_equal(to_np(counts), ref["dispatch"]["counts"])
    assert_outputs_close(y, ref["y"], "bf16", "y")


# ------------------------------------------------------------------ full-size workloads

# Threads the oracle may use over experts in the full-size checks (its
# results are the same bits for any count).
ORACLE_WORKERS = 8

# Mid-size layers that take every path at once: the three-kernel dispatch
# (more than 4096 pairs), the LDS-staged router, streaming and tiled groups
# on separate streams (a mean of 17..1023 rows per expert), the forked shared
# expert or one in the routed tile lists, fp8 128-row rest tiles and both
# weight-scale layouts.
MID = {
    "mid_zipf_bf16": get_config("prefill8192_ep8").with_(name="mid_zipf_bf16", T=4097, H=512, E=64, I=512,
                                                         I_shared=512),
    # a shared expert whose GEMM1 fills the device (16 x 16 tiles): its tiles join the routed tile lists
    "mid_shared_tiled_bf16": get_config("prefill8192_ep8").with_(name="mid_shared_tiled_bf16", T=4000, H=512,
                                                                 E=64, I=2048, I_shared=2048),
    "mid_clustered_fp8": get_config("clustered2048_fp8").with_(name="mid_clustered_fp8", T=3001, H=512, E=64,
                                                               I=2048, I_shared=2048),
    "mid_fp8_tiles": get_config("decode16_fp8").with_(name="mid_fp8_tiles", routing="zipf", T=1500, H=512, E=64,
                                                      I=2048, I_shared=2048),
}


def _full_forward(cfg):
    gin = make_inputs(cfg, DEV)
    mc = moe.cfg_from(cfg)
    y, idx, w, counts = moe.moe_forward(mc, gin.x, gin.wg, gin.bias, moe.Weights.from_inputs(gin),
                                        return_routing=True)
    torch.cuda.synchronize()
    _log(f"[full {cfg.name}] GPU forward done; oracle routing of all {cfg.T} tokens")
    r = oracle.route(oracle.to_f64(gin.x), oracle.to_f64(gin.wg), oracle.to_f64(gin.bias), cfg.k, cfg.score)
    near, mism = compare_routing(idx, w, r, cfg.k)
    if len(mism) == 0:
        np.testing.assert_array_equal(to_np(counts), np.bincount(r["idx"].ravel(), minlength=cfg.E))
    return gin, y, r, counts, near, mism


@pytest.mark.parametrize("name", ["decode16", "decode256", "decode16_fp8", "decode256_fp8"])
def test_forward_full_size_every_token(name):
    """The decode workloads at full size: every token's output, element by
    element, against the oracle computed token by token (no dispatch)."""
    cfg = get_config(name)
    _log(f"[full {name}] drawing inputs on the GPU")
    gin, y, r, counts, near, mism = _full_forward(cfg)
    toks = np.setdiff1d(np.arange(cfg.T), mism)
    _log(f"[full {name}] oracle outputs of all {len(toks)} tokens")
    yo, _ = oracle.forward_tokens(gin, toks, workers=ORACLE_WORKERS)
    err = assert_outputs_close(to_np(y)[toks], yo, tol_key(cfg), "y")
    touched = int((to_np(counts) > 0).sum())
    _log(f"[full {name}] near-ties={near} excluded={len(mism)} touched experts={touched} err={err}")
    del gin
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", sorted(MID))
def test_forward_mid_whole_layer(name):
    """The mid-size layers: the whole output against oracle.forward."""
    cfg = MID[name]
    inp, gin = _small_inputs(cfg)
    ref = oracle.forward(inp)
    y, idx, w, counts = moe.moe_forward(moe.cfg_from(cfg), gin.x, gin.wg, gin.bias, moe.Weights.from_inputs(gin),
                                        return_routing=True)
    torch.cuda.synchronize()
    near, mism = compare_routing(idx, w, ref["route"], cfg.k)
    if len(mism) == 0:
        np.testing.assert_array_equal(to_np(counts), ref["dispatch"]["counts"])
    keep = np.setdiff1d(np.arange(cfg.T), mism)
    err = assert_outputs_close(to_np(y)[keep], ref["y"][keep], tol_key(cfg), "y")
    _log(f"[mid {name}] near-ties={near} excluded={len(mism)} err={err}")


def _boundary_tokens(cfg, idx, cap=800):
    """Tokens whose rows sit where a row-position bug would show: each
    touched expert's first and last sorted slot, and the rows on both sides
    of every 256-row tile boundary and, for fp8 weights, of the 128-row rest
    tile boundary.  Taken from the oracle's dispatch of the oracle's routing."""
    d = oracle.dispatch(idx, cfg.E)
    off, sp = d["offsets"], d["sorted_pair"]
    rows = set()
    for e in range(cfg.E):
        m = int(off[e + 1] - off[e])
        if m == 0:
            continue
        cand = {0, m - 1}
        for b in range(256, m, 256):
            cand |= {b - 1, b}
        if cfg.w_dtype == "fp8" and m % 256 and m % 256 <= 128 and m > 256:
            cand |= {m - m % 256 - 1, m - m % 256}
        if m > 128:
            cand |= {127, 128}
        rows |= {int(off[e]) + r for r in cand if 0 <= r < m}
    toks = np.unique(np.asarray(sorted(sp[r] for r in rows)) // cfg.k)
    if len(toks) > cap:
        toks = np.unique(np.random.default_rng(0).choice(toks, size=cap, replace=False))
    return toks


@pytest.mark.parametrize("name", ["prefill8192_ep8", "clustered2048_fp8"])
def test_forward_full_size_boundary_tokens(name):
    """Prefill share and clustered fp8 at full size through moe_forward: the
    routing of every token, and the outputs of the tokens at every expert's
    first and last slot and at the tile boundaries."""
    cfg = get_config(name)
    _log(f"[full {name}] drawing inputs on the GPU")
    gin, y, r, counts, near, mism = _full_forward(cfg)
    toks = np.setdiff1d(_boundary_tokens(cfg, r["idx"]), mism)
    _log(f"[full {name}] oracle outputs of {len(toks)} boundary tokens")
    yo, _ = oracle.forward_tokens(gin, toks, workers=ORACLE_WORKERS)
    err = assert_outputs_close(to_np(y)[toks], yo, tol_key(cfg), "y")
    _log(f"[full {name}] near-ties={near} excluded={len(mism)} tokens={len(toks)} err={err}")
    del gin
    torch.cuda.empty_cache()


def _pick_groups(counts):
    """The largest group and one of each row class: 129..255, 33..128, 1..32."""
    counts = np.asarray(counts)
    pick = [int(np.argmax(counts))]
    for lo, hi in ((129, 255), (33, 128), (1, 32)):
        cand = [e for e in np.nonzero((counts >= lo) & (counts <= hi))[0] if e not in pick]
        if cand:
            pick.append(int(cand[len(cand) // 2]))
    return sorted(pick)


@pytest.mark.parametrize("name", ["prefill8192_ep8", "clustered2048_fp8"])
def test_expert_ffn_full_size_whole_groups(name):
    """The expert FFN at full size on the oracle's dispatch: every row of the
    largest group and of one group in each row class (129..255, 33..128 and
    1..32 rows, where the workload has one), plus the whole shared-expert
    output, element by element."""
    cfg = get_config(name)
    _log(f"[ffn {name}] drawing inputs on the GPU")
    gin = make_inputs(cfg, DEV)
    r = oracle.route(oracle.to_f64(gin.x), oracle.to_f64(gin.wg), oracle.to_f64(gin.bias), cfg.k, cfg.score)
    d = oracle.dispatch(r["idx"], cfg.E)
    off = torch.from_numpy(d["offsets"].astype(np.int32)).to(DEV)
    sp = torch.from_numpy(d["sorted_pair"].astype(np.int32)).to(DEV)
    ys, ysh = moe.moe_expert_ffn(moe.cfg_from(cfg), gin.x, off, sp, moe.Weights.from_inputs(gin))
    torch.cuda.synchronize()
    groups = _pick_groups(d["counts"])
    sizes = [int(d["counts"][e]) for e in groups]
    _log(f"[ffn {name}] oracle for groups {groups} of {sizes} rows and the shared expert")
    # the picked groups as a smaller grouped problem: group i is expert groups[i]
    full_w = oracle.OracleWeights.from_inputs(gin)
    sub_w = oracle.OracleWeights(len(groups), lambda i: full_w.expert(groups[i]), full_w.shared, full_w.fp8,
                                 full_w.block)
    segs = [d["sorted_pair"][d["offsets"][e]:d["offsets"][e + 1]] for e in groups]
    sub_off = np.concatenate([[0], np.cumsum([len(sg) for sg in segs])])
    sub_sp = np.concatenate(segs)
    xa = oracle.prepare_activations(oracle.to_f64(gin.x), full_w.fp8, full_w.block)
    ref_ys, ref_ysh = oracle.expert_ffn(xa, sub_off, sub_sp, cfg.k, sub_w)
    rows = np.concatenate([np.arange(d["offsets"][e], d["offsets"][e + 1]) for e in groups])
    key = tol_key(cfg)
    e1 = assert_outputs_close(to_np(ys)[rows], ref_ys, key, "y_sorted")
    e2 = assert_outputs_close(ysh, ref_ysh, key, "y_shared")
    _log(f"[ffn {name}] y_sorted err {e1} y_shared err {e2}")
    del gin
    torch.cuda.empty_cache()
