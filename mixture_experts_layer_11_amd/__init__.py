"""MoE-layer forward on one AMD Instinct MI355X (gfx950): HIP kernels behind a C ABI.

The library (``libmoe.so``, declared in ``include/moe.h``) implements the
DeepSeek-V3/R1 MoE layer: router (gate GEMM, scoring, selection bias, top-k,
weights), on-device dispatch (counts, offsets, stable permutation), grouped
SwiGLU experts plus the shared expert, and the weighted combine.  This package
holds the HIP sources (``csrc/``), the in-tree build and a thin ctypes binding
whose functions carry the C names.
"""

from .binding import (  # noqa: F401
    EXPORTS,
    MoeCfg,
    MoEError,
    MoEGraph,
    MoELibraryMissing,
    Weights,
    alloc_workspace,
    cfg_from,
    last_error,
    load_library,
    make_cfg,
    moe_combine,
    moe_dispatch,
    moe_expert_ffn,
    moe_expert_ffn_down,
    moe_forward,
    moe_forward_noalloc,
    moe_profile_start,
    moe_profile_stop,
    moe_quantize_fp8,
    moe_route,
    moe_routing_stats,
    moe_workspace_bytes,
    moe_workspace_ffn_h,
    status_str,
    workspace_size,
)
