"""fp64 CPU oracle of the MoE-layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library; its only common dependency is ``moe_inputs`` (seeded input
generators, which hold none of the layer's arithmetic).
"""

from .fp8 import e4m3_decode, e4m3_encode, quantize_rows_fp8  # noqa: F401
from .moe import (  # noqa: F401
    OracleWeights,
    combine,
    dispatch,
    expert_ffn,
    forward,
    forward_tokens,
    prepare_activations,
    route,
    routing_stats,
    swiglu_ffn,
    swiglu_hidden,
    to_f64,
)
