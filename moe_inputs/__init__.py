"""Seeded synthetic inputs for the MoE-layer forward.

This package holds the layer shapes (``configs``) and the random input
generators (``generate``).  It contains none of the layer's arithmetic: no
routing, no dispatch, no expert FFN, no combine.  Both the fp64 CPU oracle
(``oracle/``) and the HIP library's tests and benchmark draw their inputs from
here; nothing else is shared between them.
"""

from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
from .generate import MoEInputs, make_inputs, make_router_inputs  # noqa: F401
