"""Seeded synthetic inputs for the MoE-layer forward.

This module is the one piece shared by the HIP path's tests/bench and the
oracle: it produces inputs only and holds none of the method's arithmetic
(no routing, alignment, GEMM, activation or combine).  It does quantise the
synthetic expert weights into their storage formats, which is how inputs of
those formats are made, not a step of the layer.
"""

from .configs import CONFIGS, LayerConfig, get_config  # noqa: F401
from .generate import make_inputs, make_router_weights, make_topk_ids, make_weights, make_x, to_numpy  # noqa: F401
