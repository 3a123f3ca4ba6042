"""The C ABI from plain C: include/moe.h compiles as strict C99 with
-pedantic -Werror, and a C program linked to libmoe.so gets the same answers
as the Python binding (host-side entry points only; no GPU)."""

import os
import shutil
import subprocess

import pytest

import mixture_experts_layer_11_amd as moe
from mixture_experts_layer_11_amd import binding as B
from moe_inputs import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH) or shutil.which("gcc") is None,
                                reason="libmoe.so not built, or no gcc")


def test_c_caller(tmp_path):
    exe = tmp_path / "c_abi_check"
    libdir = os.path.dirname(B.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_abi_check.c"), "-L", libdir, "-lmoe", f"-Wl,-rpath,{libdir}",
                    "-o", str(exe)], check=True, capture_output=True, text=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True, timeout=60).stdout.splitlines()
    res = {line.split()[0]: line.split()[1:] for line in out}
    n = moe.workspace_size(B.cfg_from(CONFIGS["decode16"]))
    assert res["workspace_size"] == [str(B.MOE_OK), "MOE_OK", str(n)]
    assert res["workspace_bytes"] == [str(n)]
    h, _, _ = moe.moe_workspace_ffn_h(B.cfg_from(CONFIGS["decode16"]))
    assert res["ffn_h"] == [str(B.MOE_OK), str(h), "1", "1"]       # bf16 weights: no codes, no scales
    assert res["bad_cfg"] == [str(B.MOE_ERR_INVALID_ARG), "MOE_ERR_INVALID_ARG"]
    assert res["last_error"] == ["set"]
    assert res["forward_null_x"] == [str(B.MOE_ERR_INVALID_ARG), "MOE_ERR_INVALID_ARG"]


def _write(t, path):
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    t.numpy().tofile(path)


@pytest.mark.gpu
@pytest.mark.parametrize("w_dtype", ["bf16", "fp8"])
def test_c_forward_matches_binding(tmp_path, w_dtype):
    """The whole layer from a plain C host program (HIP runtime only, no
    torch) gives the same bits as the same call through the Python binding,
    and matches the oracle."""
    import numpy as np
    import torch

    import oracle
    from moe_inputs import get_config, make_inputs
    from parity import assert_outputs_close, compare_routing, tol_key

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    base = "decode16" if w_dtype == "bf16" else "clustered2048_fp8"
    cfg = get_config(base).with_(name=f"c_forward_{w_dtype}", routing="random", T=150, H=512, E=16, k=4, I=256,
                                 I_shared=256)
    inp = make_inputs(cfg, "cpu")
    mc = B.cfg_from(cfg)
    with open(tmp_path / "cfg.txt", "w") as f:
        f.write(" ".join(str(v) for v in (mc.T, mc.H, mc.E, mc.k, mc.I, mc.I_shared, mc.score, mc.act_dtype,
                                          mc.w_dtype, mc.quant_block, mc.w_block_rows)))
    for name, t in (("x", inp.x), ("wg", inp.wg), ("bias", inp.bias), ("w13", inp.w13), ("w2", inp.w2),
                    ("ws13", inp.ws13), ("ws2", inp.ws2), ("w13s", inp.w13_scale), ("w2s", inp.w2_scale),
                    ("ws13s", inp.ws13_scale), ("ws2s", inp.ws2_scale)):
        if t is not None:
            _write(t, tmp_path / f"{name}.bin")
    exe = tmp_path / "c_forward"
    libdir = os.path.dirname(B.LIB_PATH)
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-isystem", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c_forward.c"), "-L", libdir, "-lmoe", "-L", "/opt/rocm/lib",
                    "-lamdhip64", f"-Wl,-rpath,{libdir}", "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    print(f"[c_forward {w_dtype}] running", flush=True)
    r = subprocess.run([str(exe), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    adt = torch.bfloat16
    y_c = torch.from_numpy(np.fromfile(tmp_path / "y.bin", dtype=np.int16)).view(adt).reshape(cfg.T, cfg.H)
    idx_c = torch.from_numpy(np.fromfile(tmp_path / "idx.bin", dtype=np.int32)).reshape(cfg.T, cfg.k)

    dev = torch.device("cuda")
    w = moe.Weights(*(t.to(dev) if t is not None else None
                      for t in (inp.w13, inp.w2, inp.ws13, inp.ws2, inp.w13_scale, inp.w2_scale, inp.ws13_scale,
                                inp.ws2_scale)))
    y_b, idx_b, wt_b, _ = moe.moe_forward(mc, inp.x.to(dev), inp.wg.to(dev), inp.bias.to(dev), w,
                                          return_routing=True)
    torch.cuda.synchronize()
    assert torch.equal(idx_c, idx_b.cpu())
    assert torch.equal(y_c, y_b.cpu())
    ref = oracle.forward(inp)
    _, mism = compare_routing(idx_b, wt_b, ref["route"], cfg.k)
    keep = np.setdiff1d(np.arange(cfg.T), mism)
    assert_outputs_close(y_c[keep], ref["y"][keep], tol_key(cfg), "y")
