"""MI355X-native block-sparse masked attention (FlexAttention-style).

The compute lives in libflexattn.so (hand-written HIP kernels for gfx950,
C ABI in include/flexattn.h); ``flexattn`` is its ctypes binding and
``autotune`` picks tile shapes.
"""
from .flexattn import (  # noqa: F401
    BlockMask,
    BlockMaskT,
    FlexAttnError,
    block_mask_dims,
    build_block_mask,
    build_block_mask_t,
    bwd,
    bwd_workspace_floats,
    default_scale,
    fwd,
    load,
)
