"""MI355X (gfx950) MoE-layer forward: HIP kernels behind a C ABI (libmoe.so).

The Python side only marshals torch device tensors and the current HIP stream
into the C calls moe_route, moe_schedule and moe_forward; every step of the
layer runs in the library's kernels.
"""

from .api import (MoEBackward, MoELayer, pack_mxfp8_scales, prepare_backward, quantize_mxfp8, shape_for,  # noqa: F401
                  tile_bf16, tile_mxfp8)
