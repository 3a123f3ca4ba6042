"""Host-only checks of the C ABI (no GPU needed).

The library loads without a device; every declared symbol is exported; and
every argument error is reported by its status code before anything is
enqueued, so these calls never touch HIP.
"""

import ctypes
import os
import re

import pytest

import mixture_experts_layer_11_amd as moe
from mixture_experts_layer_11_amd import binding as B
from moe_inputs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libmoe.so not built (python -m mixture_experts_layer_11_amd.build)")


def _header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    lib = moe.load_library()
    names = _header_functions()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_status_strings():
    assert moe.status_str(B.MOE_OK) == "MOE_OK"
    assert moe.status_str(B.MOE_ERR_WORKSPACE) == "MOE_ERR_WORKSPACE"
    assert moe.status_str(99) == "MOE_ERR_UNKNOWN"


def _cfg(**kw):
    base = dict(T=16, H=7168, E=256, k=8, I=2048, I_shared=2048, score="sigmoid", act_dtype="bf16", w_dtype="bf16")
    base.update(kw)
    return B.make_cfg(**base)


def _ws_status(cfg):
    n = ctypes.c_size_t(0)
    return moe.load_library().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(n)), n.value


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_workspace_size_for_each_workload(name):
    st, n = _ws_status(B.cfg_from(CONFIGS[name]))
    assert st == B.MOE_OK and n > 0
    assert moe.moe_workspace_bytes(B.cfg_from(CONFIGS[name])) == n
    bigger = B.cfg_from(CONFIGS[name].with_(T=CONFIGS[name].T * 2))
    assert _ws_status(bigger)[1] > n


@pytest.mark.parametrize("kw,code", [
    (dict(k=0), B.MOE_ERR_INVALID_ARG),
    (dict(k=9, E=8), B.MOE_ERR_INVALID_ARG),
    (dict(T=-1), B.MOE_ERR_INVALID_ARG),
    (dict(H=0), B.MOE_ERR_INVALID_ARG),
    (dict(score=7), B.MOE_ERR_INVALID_ARG),
    (dict(E=512, k=8), B.MOE_ERR_UNSUPPORTED),
    (dict(k=33, E=64), B.MOE_ERR_UNSUPPORTED),
    (dict(H=7000), B.MOE_ERR_UNSUPPORTED),
    (dict(I=100), B.MOE_ERR_UNSUPPORTED),
    (dict(I_shared=1024), B.MOE_ERR_UNSUPPORTED),
    (dict(act_dtype="f32"), B.MOE_ERR_UNSUPPORTED),
    (dict(w_dtype="fp8", quant_block=64), B.MOE_ERR_UNSUPPORTED),
    (dict(w_dtype="fp8", I=2112), B.MOE_ERR_UNSUPPORTED),
    (dict(w_dtype="fp8", w_block_rows=64), B.MOE_ERR_UNSUPPORTED),
    (dict(n_group=3, topk_group=1), B.MOE_ERR_INVALID_ARG),              # E = 256 not a multiple of 3
    (dict(n_group=8, topk_group=9), B.MOE_ERR_INVALID_ARG),              # topk_group > n_group
    (dict(n_group=8, topk_group=0), B.MOE_ERR_INVALID_ARG),
    (dict(n_group=128, topk_group=4), B.MOE_ERR_UNSUPPORTED),            # valid, but more than 64 groups
    (dict(n_group=256, topk_group=8), B.MOE_ERR_INVALID_ARG),            # groups of one expert
    (dict(E=16, n_group=8, topk_group=1, k=4), B.MOE_ERR_INVALID_ARG),   # k above the eligible experts
])
def test_invalid_configs_rejected(kw, code):
    st, _ = _ws_status(_cfg(**kw))
    assert st == code, moe.last_error()
    assert moe.last_error()
    assert moe.moe_workspace_bytes(_cfg(**kw)) == 0
    assert moe.last_error()


@pytest.mark.parametrize("name", sorted(CONFIGS))
def test_workspace_ffn_h_regions(name):
    """h (and for fp8 its codes and scales) lie inside the workspace, apart."""
    c = CONFIGS[name]
    cfg = B.cfg_from(c)
    h, hq, hs = moe.moe_workspace_ffn_h(cfg)
    rows = c.T * c.k + (c.T if c.I_shared else 0)
    esz = 2 if c.w_dtype == "bf16" else 4
    regions = [(h, rows * c.I * esz)]
    if c.w_dtype == "fp8":
        regions += [(hq, rows * c.I), (hs, rows * (c.I // c.quant_block) * 4)]
    else:
        assert hq is None and hs is None
    regions.sort()
    assert all(off % 256 == 0 for off, _ in regions)
    for (a, n), (b, _) in zip(regions, regions[1:]):
        assert a + n <= b
    assert regions[-1][0] + regions[-1][1] <= moe.moe_workspace_bytes(cfg)


def test_workspace_ffn_h_errors():
    lib = moe.load_library()
    assert moe.moe_workspace_ffn_h(_cfg(T=0)) == (None, None, None)
    n = ctypes.c_size_t(0)
    assert lib.moe_workspace_ffn_h(ctypes.byref(_cfg()), ctypes.byref(n), None, ctypes.byref(n)) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_workspace_ffn_h(ctypes.byref(_cfg(k=0)), ctypes.byref(n), ctypes.byref(n),
                                   ctypes.byref(n)) == B.MOE_ERR_INVALID_ARG


def test_workspace_bytes_null_cfg_and_tiny_layer():
    lib = moe.load_library()
    assert lib.moe_workspace_bytes(None) == 0 and "cfg" in moe.last_error()
    n = moe.moe_workspace_bytes(_cfg(T=0))          # valid, nothing to hold: still nonzero
    assert n > 0 and moe.last_error() == ""


def test_argument_errors_before_any_launch():
    lib = moe.load_library()
    cfg = _cfg()
    _, need = _ws_status(cfg)
    fake = 1 << 20                       # never dereferenced: validation fails first
    byref = ctypes.byref
    # null required pointer
    assert lib.moe_route(byref(cfg), None, fake, None, fake, fake, fake, need, None) == B.MOE_ERR_INVALID_ARG
    assert "x" in moe.last_error()
    # misaligned pointer
    assert lib.moe_route(byref(cfg), fake + 2, fake, None, fake, fake, fake, need, None) == B.MOE_ERR_INVALID_ARG
    # workspace too small
    assert lib.moe_route(byref(cfg), fake, fake, None, fake, fake, fake, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_dispatch(byref(cfg), fake, fake, fake, fake, fake, fake, 0, None) == B.MOE_ERR_WORKSPACE
    # null cfg
    assert lib.moe_forward(None, fake, fake, None, None, fake, None, None, None, fake, need, None) == B.MOE_ERR_INVALID_ARG
    # missing weights / shared-expert output inconsistency
    w = B.MoeWeights(fake, None, fake, None, None, None, None, None)
    assert lib.moe_expert_ffn(byref(cfg), fake, fake, fake, byref(w), fake, fake, fake, need, None) == B.MOE_ERR_INVALID_ARG
    cfg_ns = _cfg(I_shared=0)
    _, need_ns = _ws_status(cfg_ns)
    assert lib.moe_expert_ffn(byref(cfg_ns), fake, fake, fake, byref(w), fake, fake, fake, need_ns, None) == B.MOE_ERR_INVALID_ARG
    # fp8 weights without scales
    cfg8 = _cfg(w_dtype="fp8")
    _, need8 = _ws_status(cfg8)
    w8 = B.MoeWeights(fake, None, fake, None, fake, fake, fake, fake)
    assert lib.moe_expert_ffn(byref(cfg8), fake, fake, fake, byref(w8), fake, fake, fake, need8, None) == B.MOE_ERR_INVALID_ARG
    # down projection alone: x is not an argument; the same checks as moe_expert_ffn otherwise
    wf = B.MoeWeights(fake, None, fake, None, fake, None, fake, None)
    assert lib.moe_expert_ffn_down(byref(cfg), None, fake, byref(wf), fake, fake, fake, need, None) == B.MOE_ERR_INVALID_ARG
    assert "offsets" in moe.last_error()
    assert lib.moe_expert_ffn_down(byref(cfg), fake, fake, byref(w), fake, fake, fake, need, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn_down(byref(cfg), fake, fake, byref(wf), fake, fake, fake, need - 1, None) == B.MOE_ERR_WORKSPACE
    assert lib.moe_expert_ffn_down(byref(cfg8), fake, fake, byref(w8), fake, fake, fake, need8, None) == B.MOE_ERR_INVALID_ARG
    # combine: bad pointers
    assert lib.moe_combine(byref(cfg), None, None, fake, fake, fake, None) == B.MOE_ERR_INVALID_ARG
    # quantiser: bad block / shape
    assert lib.moe_quantize_fp8(4, 100, 128, fake, B.MOE_BF16, fake, fake, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_fp8(4, 512, 100, fake, B.MOE_BF16, fake, fake, None) == B.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_fp8(4, 512, 128, fake, B.MOE_FP8_E4M3, fake, fake, None) == B.MOE_ERR_UNSUPPORTED


def test_zero_tokens_is_a_no_op():
    lib = moe.load_library()
    cfg = _cfg(T=0)
    byref = ctypes.byref
    assert lib.moe_route(byref(cfg), None, None, None, None, None, None, 0, None) == B.MOE_OK
    assert lib.moe_dispatch(byref(cfg), None, None, None, None, None, None, 0, None) == B.MOE_OK
    assert lib.moe_combine(byref(cfg), None, None, None, None, None, None) == B.MOE_OK
    assert lib.moe_expert_ffn_down(byref(cfg), None, None, None, None, None, None, 0, None) == B.MOE_OK
    assert lib.moe_forward(byref(cfg), None, None, None, None, None, None, None, None, None, 0, None) == B.MOE_OK
    assert lib.moe_quantize_fp8(0, 128, 128, None, B.MOE_BF16, None, None, None) == B.MOE_OK


def test_binding_raises_typed_errors():
    with pytest.raises(moe.MoEError) as ei:
        moe.workspace_size(_cfg(k=0))
    assert ei.value.status == B.MOE_ERR_INVALID_ARG


def test_graph_entry_points_validate_before_any_hip_call():
    lib = moe.load_library()
    cfg = _cfg()
    _, need = _ws_status(cfg)
    fake = 1 << 20
    h = ctypes.c_void_p(123)
    w = B.MoeWeights()
    # no output handle
    assert lib.moe_graph_capture(ctypes.byref(cfg), fake, fake, None, ctypes.byref(w), fake, None, None, None, fake,
                                 need, None, None) == B.MOE_ERR_INVALID_ARG
    # T = 0: nothing to capture; the handle is cleared
    zero = _cfg(T=0)
    assert lib.moe_graph_capture(ctypes.byref(zero), fake, fake, None, ctypes.byref(w), fake, None, None, None, fake,
                                 need, None, ctypes.byref(h)) == B.MOE_ERR_INVALID_ARG
    assert not h.value
    # argument errors surface from the eager call's validation, before any launch
    assert lib.moe_graph_capture(ctypes.byref(cfg), None, fake, None, ctypes.byref(w), fake, None, None, None, fake,
                                 need, None, ctypes.byref(h)) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_graph_capture(ctypes.byref(_cfg(k=0)), fake, fake, None, ctypes.byref(w), fake, None, None, None,
                                 fake, need, None, ctypes.byref(h)) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_graph_launch(None, None) == B.MOE_ERR_INVALID_ARG
    assert lib.moe_graph_destroy(None) == B.MOE_OK
