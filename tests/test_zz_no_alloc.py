"""moe_forward_noalloc, the entry point for callers that cannot allocate,
against moe_forward (which takes a workspace): the same kernels, so the same
bits.  Two calls in a row on the same scratch, the second on a smaller
input, for a bf16 and an fp8 decode layer and for a bf16 and an fp8 layer
that takes every FFN path; and a layer above the scratch's fixed size is
refused before anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

import mixture_experts_layer_11_amd as moe
from mixture_experts_layer_11_amd import binding as B
from moe_inputs import get_config, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu_and_library():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    moe.load_library()


def _outputs(cfg):
    adt = torch.float32 if cfg.act_dtype == "f32" else torch.bfloat16
    return (torch.full((cfg.T, cfg.H), float("nan"), dtype=adt, device=DEV),
            torch.full((cfg.T, cfg.k), -5, dtype=torch.int32, device=DEV),
            torch.full((cfg.T, cfg.k), float("nan"), dtype=torch.float32, device=DEV),
            torch.full((cfg.E,), -5, dtype=torch.int32, device=DEV))


def _check_pair(cfg, inp, x):
    mc = moe.cfg_from(cfg)
    w = moe.Weights.from_inputs(inp)
    y, idx, wt, counts = _outputs(cfg)
    moe.moe_forward_noalloc(mc, x, inp.wg, inp.bias, w, y, idx, wt, counts)
    ref = moe.moe_forward(mc, x, inp.wg, inp.bias, w, return_routing=True)
    torch.cuda.synchronize()
    for name, a, b in zip(("y", "topk_idx", "topk_w", "counts"), (y, idx, wt, counts), ref):
        assert torch.equal(a, b), f"{cfg.name} T={cfg.T}: {name} differs from moe_forward"
    print(f"[noalloc] {cfg.name} T={cfg.T}: equal to moe_forward, scratch {moe.moe_workspace_bytes(mc) >> 20} MiB",
          flush=True)


@pytest.mark.parametrize("name,small_T", [("decode256", 16), ("decode256_fp8", 24)])
def test_noalloc_equals_forward_twice_second_smaller(name, small_T):
    cfg = get_config(name)
    print(f"[noalloc] drawing {name}", flush=True)
    inp = make_inputs(cfg, DEV)
    _check_pair(cfg, inp, inp.x)
    # the same layer on fewer tokens: the scratch keeps the first call's contents
    small = cfg.with_(T=small_T)
    _check_pair(small, inp, inp.x[:small_T].contiguous())
    del inp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("base", ["decode16", "clustered2048_fp8"])
def test_noalloc_small_layers_with_shared_fork_paths(base):
    """A layer whose moe_forward forks the shared expert and the tiled groups
    onto side streams; the no-allocation call keeps everything on one stream
    and must still give the same bits.  In fp8 the first call's routed tiles
    quantise h in their epilogue (75 rows per expert on average) and the
    second call's do not (12.5)."""
    cfg = get_config(base).with_(name=f"noalloc_both_{base}", routing="zipf", T=600, H=1024, E=32, k=4, I=256,
                                 I_shared=256)
    inp = make_inputs(cfg, DEV)
    _check_pair(cfg, inp, inp.x)
    _check_pair(cfg.with_(T=100), inp, inp.x[:100].contiguous())


def test_noalloc_refuses_a_layer_above_the_scratch():
    cfg = moe.cfg_from(get_config("prefill8192_ep8"))
    assert moe.moe_workspace_bytes(cfg) > 64 << 20
    fake = 1 << 20                       # never dereferenced: refused before any launch
    w = B.MoeWeights(fake, None, fake, None, fake, None, fake, None)
    st = moe.load_library().moe_forward_noalloc(ctypes.byref(cfg), fake, fake, None, ctypes.byref(w), fake, None,
                                                None, None, None)
    assert st == B.MOE_ERR_WORKSPACE and "scratch" in moe.last_error()
