"""DeepSeekMoE layer forward on MI355X (gfx950): Python binding of libmoe.so.

The layer's work runs in the HIP kernels of libmoe.so, reached through the C
ABI in include/moe.h; this package only marshals torch tensors to it.
"""
from . import ops  # noqa: F401
from ._lib import LIB_PATH, MoeError, lib  # noqa: F401
from .ops import (  # noqa: F401
    Forward, Layer, combine, expert_ffn, forward, pack_weights, permute, route, route_noisy, route_stats,
    shared_ffn, split_stats,
)
