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
