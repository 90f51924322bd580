"""MI355X-native DSpark/DFlash draft-block forward (Eq 2 + Eq 3).

The compute lives in libdspark.so (hand-written HIP for gfx950 behind the C
ABI of include/dspark.h); this package is its Python binding.
"""
from .api import (DsparkDims, DsparkError, PreparedForward, block_forward, block_layer,  # noqa: F401
                  block_layer_noalloc,
                  ctx_fuse, kernel_names, plan_info, trace_begin, trace_end, version,
                  workspace_size)
from ._lib import OP_BLOCK_FORWARD, OP_BLOCK_LAYER, OP_CTX_FUSE  # noqa: F401
