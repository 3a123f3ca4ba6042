"""Host logic of bench.py (no GPU): the algorithmic byte and FLOP model
that the roofline fractions divide by, and the refusal of more than one GPU."""

import os
import subprocess
import sys

import bench
from moe_inputs import get_config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _weights_bytes(cfg):
    return 3 * cfg.H * cfg.I * 2


def test_halves_mode_books_the_shared_expert_under_the_streaming_kernel():
    """T <= 16: the shared expert runs as two 8-row halves inside the routed
    streaming launch, so its weight bytes belong to ffn_gemm{1,2}_skinny."""
    cfg = get_config("decode16")
    counts = [0] * cfg.E
    for e in range(cfg.T * cfg.k):
        counts[e % 100] += 1                   # 100 touched experts of 1-2 rows
    models, layer = bench.kernel_models(cfg, counts)
    H, I = cfg.H, cfg.I
    g1 = models["ffn_gemm1_skinny"]["bytes"]
    g2 = models["ffn_gemm2_skinny"]["bytes"]
    assert models["ffn_gemm1_shared_skinny"]["bytes"] == 0
    # 101 weight sets (100 routed + shared) read once each
    assert g1 >= 101 * 2 * I * H * 2 and g2 >= 101 * H * I * 2
    rows = cfg.T * cfg.k + cfg.T
    assert g1 == 101 * 2 * I * H * 2 + rows * H * 2 + rows * I * 2
    assert layer["touched"] == 100
    assert models["ffn_gemm1_skinny"]["flops"] == 2 * rows * 2 * I * H


def test_shared_expert_has_its_own_launch_from_17_tokens():
    cfg = get_config("decode16").with_(T=24)
    counts = [1] * (cfg.T * cfg.k) + [0] * (cfg.E - cfg.T * cfg.k)
    models, _ = bench.kernel_models(cfg, counts)
    assert models["ffn_gemm1_shared_skinny"]["bytes"] == 2 * cfg.I * cfg.H * 2 + cfg.T * cfg.H * 2 + cfg.T * cfg.I * 2


def test_prefill_layer_model():
    """Every group of the prefill share is tiled; the layer's FLOPs are
    (P + T) * 6 H I + 2 T H E and its bytes the touched weights once, the
    gate and bias, and x and y."""
    cfg = get_config("prefill8192_ep8")
    counts = [cfg.T * cfg.k // cfg.E] * cfg.E
    models, layer = bench.kernel_models(cfg, counts)
    P, T, H, I, E = cfg.T * cfg.k, cfg.T, cfg.H, cfg.I, cfg.E
    assert layer["flops"] == (P + T) * 6 * H * I + 2 * T * H * E
    assert layer["bytes"] == (E + 1) * _weights_bytes(cfg) + E * H * 2 + E * 4 + 2 * T * H * 2
    # the shared expert's GEMM1 (32 x 16 tiles) fills the device: its tiles run in the routed launches
    assert bench.shared_in_lists(cfg)
    assert models["ffn_gemm1_tiled"]["flops"] == 2 * (P + T) * 2 * I * H
    assert models["ffn_gemm1_shared_tiled"]["flops"] == 0
    assert models["ffn_gemm1_skinny"]["bytes"] == 0
    assert not bench.shares_device(cfg)
    assert bench.shares_device(get_config("clustered2048_fp8"))
    assert not bench.shares_device(get_config("decode256"))
    assert not bench.shared_in_lists(get_config("decode256"))
    assert not bench.shared_in_lists(get_config("clustered2048_fp8"))


def test_fp8_routed_tiles_write_h_codes_and_scales():
    """fp8: a routed group of 33..128 rows takes one 128-row tile, whose GEMM1
    writes h's E4M3 codes and one fp32 scale per 128 values; a streaming
    group writes fp32 h (quantised by a separate launch); the shared expert's
    own tiles write fp32 h."""
    cfg = get_config("clustered2048_fp8")
    H, I, qb = cfg.H, cfg.I, cfg.quant_block
    w13 = 2 * I * H + (2 * I) * (H // qb) * 4            # codes and 1 x 128 scales
    counts = [100, 20] + [0] * (cfg.E - 2)
    models, _ = bench.kernel_models(cfg.with_(I_shared=0), counts)
    assert models["ffn_gemm1_tiled128"]["bytes"] == w13 + 100 * H + 100 * H // qb * 4 + 100 * I + 100 * I // qb * 4
    assert models["ffn_gemm1_skinny"]["bytes"] == w13 + 20 * H + 20 * H // qb * 4 + 20 * I * 4
    models, _ = bench.kernel_models(cfg, [0] * cfg.E)
    T = cfg.T
    assert models["ffn_gemm1_shared_tiled"]["bytes"] == w13 + T * H + T * H // qb * 4 + T * I * 4
    # a few rows per expert on average (decode256_fp8): any tile writes fp32 h
    dcfg = get_config("decode256_fp8").with_(I_shared=0)
    models, _ = bench.kernel_models(dcfg, [100] + [0] * (dcfg.E - 1))
    w13d = 2 * I * H + (2 * I // dcfg.w_block_rows) * (H // qb) * 4
    assert models["ffn_gemm1_tiled128"]["bytes"] == w13d + 100 * H + 100 * H // qb * 4 + 100 * I * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
