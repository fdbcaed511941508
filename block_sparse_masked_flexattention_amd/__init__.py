"""MI355X-native block-sparse masked attention forward (FlexAttention-style).

The compute lives in libflexattn.so (hand-written HIP kernels for gfx950,
C ABI in include/flexattn.h); ``flexattn`` is its ctypes binding.
"""
from .flexattn import (  # noqa: F401
    BlockMask,
    FlexAttnError,
    block_mask_dims,
    build_block_mask,
    default_scale,
    fwd,
    load,
)
