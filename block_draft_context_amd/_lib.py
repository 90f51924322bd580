"""ctypes view of libdspark.so (include/dspark.h)."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdspark.so")

OK, EINVAL, EUNSUPPORTED, EWORKSPACE, EHIP = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
OP_CTX_FUSE, OP_BLOCK_LAYER, OP_BLOCK_FORWARD, OP_CTX_APPEND, OP_BLOCK_PROPOSE = 0, 1, 2, 3, 4
NOALLOC_SCRATCH_BYTES = 64 << 20   # the no-allocation entry point's device array

# every function the header declares
EXPORTS = [
    "dspark_workspace_size", "dspark_ctx_fuse", "dspark_block_layer",
    "dspark_block_forward", "dspark_last_error", "dspark_version",
    "dspark_kernel_kinds", "dspark_kernel_name", "dspark_trace_begin",
    "dspark_trace_end", "dspark_plan_info", "dspark_block_layer_noalloc",
    "dspark_cache_bytes", "dspark_cache_reset", "dspark_ctx_append", "dspark_block_propose",
    "dspark_markov_workspace_size", "dspark_markov_draft", "dspark_block_build",
    "dspark_padded_workspace_size", "dspark_block_forward_padded",
]
PLAN_FIELDS = ("ctx_splits", "ctx_k_per_split", "attn_chunk", "attn_tiles", "attn_streaming",
               "workspace_bytes", "ctx_fused_norm", "ctx_tail_rows")


QK_NORM, PLAIN_CTX_KV, GELU_FFN = 1, 2, 4   # dspark_variant bits


class Dims(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("H", ctypes.c_int32), ("d", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("gamma", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("ff", ctypes.c_int32),
                ("eps", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("variant", ctypes.c_int32),
                ("rope_theta", ctypes.c_float)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "attn_norm", "wq", "wk", "wv", "wo", "ff_norm", "w_gate", "w_up", "w_down",
        "q_norm", "k_norm")]


class DsparkError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dspark status {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m block_draft_context_amd.build` "
            "(or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pi32 = ctypes.POINTER(ctypes.c_int32)
    L.dspark_workspace_size.argtypes = [i32, ctypes.POINTER(Dims), i32, pi32]
    L.dspark_workspace_size.restype = sz
    L.dspark_ctx_fuse.argtypes = [ctypes.POINTER(Dims), i32, pi32, vp, ctypes.POINTER(vp), i64,
                                  vp, vp, vp, vp, sz, vp]
    L.dspark_ctx_fuse.restype = i32
    L.dspark_block_layer.argtypes = [ctypes.POINTER(Dims), i32, pi32, vp, vp, vp, vp,
                                     ctypes.POINTER(LayerWeights), vp, sz, vp]
    L.dspark_block_layer.restype = i32
    L.dspark_block_forward.argtypes = [ctypes.POINTER(Dims), i32, pi32, vp, ctypes.POINTER(vp), i64,
                                       vp, vp, vp, vp, ctypes.POINTER(LayerWeights), vp, vp, vp,
                                       vp, sz, vp]
    L.dspark_block_forward.restype = i32
    L.dspark_last_error.argtypes = []
    L.dspark_last_error.restype = ctypes.c_char_p
    L.dspark_version.argtypes = []
    L.dspark_version.restype = ctypes.c_char_p
    L.dspark_kernel_kinds.argtypes = []
    L.dspark_kernel_kinds.restype = i32
    L.dspark_kernel_name.argtypes = [i32]
    L.dspark_kernel_name.restype = ctypes.c_char_p
    L.dspark_trace_begin.argtypes = [ctypes.c_uint64, i32]
    L.dspark_trace_begin.restype = i32
    L.dspark_trace_end.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64), i32]
    L.dspark_trace_end.restype = i32
    L.dspark_block_layer_noalloc.argtypes = [ctypes.POINTER(Dims), i32, pi32, vp, vp, vp, vp,
                                             ctypes.POINTER(LayerWeights), vp]
    L.dspark_block_layer_noalloc.restype = i32
    L.dspark_cache_bytes.argtypes = [ctypes.POINTER(Dims), i32, i32]
    L.dspark_cache_bytes.restype = sz
    L.dspark_cache_reset.argtypes = [ctypes.POINTER(Dims), i32, i32, vp, vp]
    L.dspark_cache_reset.restype = i32
    L.dspark_ctx_append.argtypes = [ctypes.POINTER(Dims), i32, i32, pi32, vp, pi32, vp,
                                    ctypes.POINTER(vp), i64, vp, vp, ctypes.POINTER(LayerWeights),
                                    vp, vp, sz, vp]
    L.dspark_ctx_append.restype = i32
    L.dspark_block_propose.argtypes = [ctypes.POINTER(Dims), i32, i32, pi32, vp, vp, vp, vp,
                                       ctypes.POINTER(LayerWeights), vp, vp, vp, sz, vp]
    L.dspark_block_propose.restype = i32
    L.dspark_markov_workspace_size.argtypes = [ctypes.POINTER(Dims), i32, i32, i32]
    L.dspark_markov_workspace_size.restype = sz
    L.dspark_markov_draft.argtypes = [ctypes.POINTER(Dims), i32, i32, i32] + [vp] * 11 + [sz, vp]
    L.dspark_markov_draft.restype = i32
    L.dspark_block_build.argtypes = [ctypes.POINTER(Dims), i32, vp, vp, vp, vp, vp]
    L.dspark_block_build.restype = i32
    L.dspark_padded_workspace_size.argtypes = [ctypes.POINTER(Dims), i32, i32]
    L.dspark_padded_workspace_size.restype = sz
    L.dspark_block_forward_padded.argtypes = [ctypes.POINTER(Dims), i32, i32, ctypes.POINTER(vp), i64,
                                              vp, vp, vp, vp, vp, ctypes.POINTER(LayerWeights), vp, vp,
                                              vp, vp, sz, vp]
    L.dspark_block_forward_padded.restype = i32
    L.dspark_plan_info.argtypes = [i32, ctypes.POINTER(Dims), i32, pi32, ctypes.POINTER(ctypes.c_int64), i32]
    L.dspark_plan_info.restype = i32
    _lib = L
    return L


def check(status: int) -> None:
    if status != OK:
        raise DsparkError(status, lib().dspark_last_error().decode(errors="replace"))
