"""Prism dynamic sparse video self-attention for MI355X (gfx950).

The compute lives in libprism.so (hand-written HIP kernels behind the C ABI
declared in include/prism.h); this package holds its ctypes binding
(`binding`), the device-buffer helper (`pipeline`) and the build script
(`build`).
"""

from . import binding  # noqa: F401
from .binding import (make_params, make_problem, prism_attn_bwd, prism_attn_fwd,  # noqa: F401
                      prism_dense_attn_bwd, prism_dense_attn_fwd, prism_plan_shapes, prism_select_blocks,
                      prism_zone_stats)
