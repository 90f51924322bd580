"""MI355X-native DSpark/DFlash draft-block forward (Eq 2 + Eq 3).

The compute lives in libdspark.so (hand-written HIP for gfx950 behind the C
ABI of include/dspark.h); this package is its Python binding.
"""
from .api import (DraftCache, DsparkDims, DsparkError, PreparedForward, block_build,  # noqa: F401
                  block_forward, block_forward_padded,
                  block_layer, block_layer_noalloc, cache_bytes, markov_draft, markov_workspace_size,
                  padded_workspace_size, prepared_append,
                  prepared_propose,
                  ctx_fuse, kernel_names, plan_info, trace_begin, trace_end, version,
                  workspace_size)
from ._lib import (OP_BLOCK_FORWARD, OP_BLOCK_LAYER, OP_BLOCK_PROPOSE, OP_CTX_APPEND,  # noqa: F401
                   OP_CTX_FUSE)
