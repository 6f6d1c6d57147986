"""Single-GPU Mixture-of-Experts layer forward for AMD Instinct MI355X
(gfx950): HIP kernels behind the C ABI of include/moe.h (libmoe.so) and a
thin torch binding with the same names."""

from ._lib import LIB_PATH, MoeError, lib  # noqa: F401
from .ops import (align, align_max_blocks, align_max_padded, debug_error, expert_ffn,  # noqa: F401
                  layer, layer_block_m, layer_noalloc, layer_workspace_size, probe_empty, probe_mfma, probe_read, route, route_align,
                  workspace)
