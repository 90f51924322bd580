"""Python binding of the C ABI (include/dspark.h): argument marshalling only.

Every step of the forward runs in libdspark.so. torch supplies device memory
and the current HIP stream; nothing here computes the method. Outputs and the
workspace are allocated with torch when the caller does not pass them.

Matrices are passed as the library takes them: row-major [out, in] (y = x W^T),
W_c as [d, m*H] and the layer matrices as wq/wk/wv/wo [d, d], w_gate/w_up
[ff, d], w_down [d, ff].
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Dict, List, Optional, Sequence

import torch

from . import _lib as L

__all__ = [
    "DsparkDims", "workspace_size", "ctx_fuse", "block_layer", "block_forward",
    "version", "kernel_names", "trace_begin", "trace_end", "DsparkError", "PreparedForward",
    "plan_info", "block_layer_noalloc", "cache_bytes", "DraftCache", "PreparedCall",
    "prepared_propose", "prepared_append", "markov_draft", "block_build", "block_forward_padded",
]

DsparkError = L.DsparkError

_TORCH_DTYPE = {L.F32: torch.float32, L.BF16: torch.bfloat16}
LAYER_KEYS = ("attn_norm", "wq", "wk", "wv", "wo", "ff_norm", "w_gate", "w_up", "w_down",
              "q_norm", "k_norm")


@dataclasses.dataclass
class DsparkDims:
    m: int
    H: int
    d: int
    n_heads: int
    gamma: int
    n_layers: int
    ff: int
    eps: float = 1e-6
    dtype: str = "bf16"      # "bf16" or "f32": storage of the long tensors
    n_kv_heads: int = 0      # 0 = n_heads
    qk_norm: bool = False    # variant switches (include/dspark.h, dspark_variant)
    plain_ctx_kv: bool = False
    gelu_ffn: bool = False
    rope_theta: float = 0.0

    @property
    def code(self) -> int:
        return {"f32": L.F32, "bf16": L.BF16}[self.dtype]

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.code]

    @property
    def variant(self) -> int:
        return ((L.QK_NORM if self.qk_norm else 0) | (L.PLAIN_CTX_KV if self.plain_ctx_kv else 0)
                | (L.GELU_FFN if self.gelu_ffn else 0))

    def c(self) -> L.Dims:
        return L.Dims(self.m, self.H, self.d, self.n_heads, self.gamma, self.n_layers, self.ff,
                      float(self.eps), self.code, int(self.n_kv_heads), self.variant,
                      float(self.rope_theta))


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _cu_host(cu) -> ctypes.Array:
    vals = [int(v) for v in (cu.tolist() if hasattr(cu, "tolist") else cu)]
    return (ctypes.c_int32 * len(vals))(*vals)


def _torch_stream(stream) -> "torch.cuda.Stream":
    """The stream the library enqueues on, as a torch stream object: the
    current one for None, the given one, or a raw hipStream_t handle wrapped
    as an external stream. Outputs and workspaces that this module allocates
    are allocated on it (``with torch.cuda.stream``), so the caching
    allocator never hands their memory to other work before the library's
    kernels on that stream are done with it."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _stream(stream) -> int:
    return _torch_stream(stream).cuda_stream


def version() -> str:
    return L.lib().dspark_version().decode()


def kernel_names() -> List[str]:
    lib = L.lib()
    return [lib.dspark_kernel_name(i).decode() for i in range(lib.dspark_kernel_kinds())]


def workspace_size(op: int, dims: DsparkDims, cu) -> int:
    cu_h = _cu_host(cu)
    A = len(cu_h) - 1
    dm = dims.c()
    n = L.lib().dspark_workspace_size(op, ctypes.byref(dm), A, cu_h)
    if n == 0:
        raise DsparkError(L.EINVAL, L.lib().dspark_last_error().decode(errors="replace"))
    return int(n)


def plan_info(op: int, dims: DsparkDims, cu) -> Dict[str, int]:
    """The launch plan the library takes for these sizes (host arithmetic)."""
    cu_h = _cu_host(cu)
    dm = dims.c()
    out = (ctypes.c_int64 * len(L.PLAN_FIELDS))()
    n = L.lib().dspark_plan_info(op, ctypes.byref(dm), len(cu_h) - 1, cu_h, out, len(out))
    if n == 0:
        raise DsparkError(L.EINVAL, L.lib().dspark_last_error().decode(errors="replace"))
    return {k: int(out[i]) for i, k in enumerate(L.PLAN_FIELDS[:n])}


def _workspace(op, dims, cu, ws, device):
    need = workspace_size(op, dims, cu)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def _tap_list(taps, dims: "DsparkDims") -> List[torch.Tensor]:
    """The m taps as [T, H] views; they must share the storage dtype and one
    row stride (the library takes a single leading dimension)."""
    if isinstance(taps, torch.Tensor):
        taps = list(taps.unbind(0))
    taps = list(taps)
    if len(taps) != dims.m:
        raise ValueError(f"{len(taps)} taps given, dims.m = {dims.m}")
    ld = int(taps[0].stride(0))
    for j, t in enumerate(taps):
        if t.dtype != dims.torch_dtype:
            raise ValueError(f"taps[{j}] is {t.dtype}, the storage dtype is {dims.torch_dtype}")
        if t.dim() != 2 or t.stride(1) != 1 or int(t.stride(0)) != ld:
            raise ValueError(f"taps[{j}] must be a row-major [T, H] view with row stride {ld}")
    return taps


def _tap_ptrs(taps) -> ctypes.Array:
    return (ctypes.c_void_p * len(taps))(*[t.data_ptr() for t in taps])


def _tap_ld(taps) -> int:
    return int(taps[0].stride(0))


def _cu_dev(cu, cu_dev, device):
    if cu_dev is not None:
        return cu_dev
    return torch.as_tensor([int(v) for v in (cu.tolist() if hasattr(cu, "tolist") else cu)],
                           dtype=torch.int32, device=device)


def _layer_struct(lw: Dict[str, torch.Tensor]) -> L.LayerWeights:
    return L.LayerWeights(*[_ptr(lw.get(k)) for k in LAYER_KEYS])


def ctx_fuse(dims: DsparkDims, cu, taps, w_c, ctx_norm, *, cu_dev=None, h_ctx=None, ws=None,
             stream=None) -> torch.Tensor:
    """Eq 2: H_ctx [T, d] from the m tapped hidden states (list of [T, H] or [m, T, H])."""
    device = w_c.device
    cu_h = _cu_host(cu)
    T = cu_h[len(cu_h) - 1]
    taps = _tap_list(taps, dims)
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if h_ctx is None:
            h_ctx = torch.empty((T, dims.d), dtype=dims.torch_dtype, device=device)
        cu_dev = _cu_dev(cu, cu_dev, device)
        ws, nbytes = _workspace(L.OP_CTX_FUSE, dims, cu, ws, device)
    dm = dims.c()
    L.check(L.lib().dspark_ctx_fuse(ctypes.byref(dm), len(cu_h) - 1, cu_h, _ptr(cu_dev),
                                    _tap_ptrs(taps), _tap_ld(taps), _ptr(w_c), _ptr(ctx_norm),
                                    _ptr(h_ctx), _ptr(ws), nbytes, ts.cuda_stream))
    return h_ctx


def block_layer(dims: DsparkDims, cu, h_ctx, d_in, lw: Dict[str, torch.Tensor], *, cu_dev=None,
                d_out=None, ws=None, stream=None) -> torch.Tensor:
    """Eq 3 + FFN for one draft layer: block rows [A, gamma, d] float32 in and out."""
    device = d_in.device
    cu_h = _cu_host(cu)
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if d_out is None:
            d_out = torch.empty_like(d_in)
        cu_dev = _cu_dev(cu, cu_dev, device)
        ws, nbytes = _workspace(L.OP_BLOCK_LAYER, dims, cu, ws, device)
    dm = dims.c()
    lws = _layer_struct(lw)
    L.check(L.lib().dspark_block_layer(ctypes.byref(dm), len(cu_h) - 1, cu_h, _ptr(cu_dev),
                                       _ptr(h_ctx), _ptr(d_in), _ptr(d_out), ctypes.byref(lws),
                                       _ptr(ws), nbytes, ts.cuda_stream))
    return d_out


def block_layer_noalloc(dims: DsparkDims, cu, h_ctx, d_in, lw: Dict[str, torch.Tensor], *,
                        cu_dev, d_out, stream=None) -> torch.Tensor:
    """block_layer with the library's own device scratch: the library call
    allocates nothing. The caller passes the device copy of cu and the
    output; calls on one GPU must not overlap."""
    cu_h = _cu_host(cu)
    dm = dims.c()
    lws = _layer_struct(lw)
    L.check(L.lib().dspark_block_layer_noalloc(ctypes.byref(dm), len(cu_h) - 1, cu_h, _ptr(cu_dev),
                                               _ptr(h_ctx), _ptr(d_in), _ptr(d_out),
                                               ctypes.byref(lws), _stream(stream)))
    return d_out


def block_forward(dims: DsparkDims, cu, taps, w_c, ctx_norm, block_in, block_pos,
                  layers: Sequence[Dict[str, torch.Tensor]], out_norm=None, *, cu_dev=None,
                  h_ctx_out=None, block_out=None, ws=None, stream=None) -> torch.Tensor:
    """The whole draft block (Eq 2, block init, every layer, output norm)."""
    device = block_in.device
    cu_h = _cu_host(cu)
    taps = _tap_list(taps, dims)
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if block_out is None:
            block_out = torch.empty_like(block_in)
        cu_dev = _cu_dev(cu, cu_dev, device)
        ws, nbytes = _workspace(L.OP_BLOCK_FORWARD, dims, cu, ws, device)
    dm = dims.c()
    arr = (L.LayerWeights * len(layers))(*[_layer_struct(lw) for lw in layers])
    L.check(L.lib().dspark_block_forward(
        ctypes.byref(dm), len(cu_h) - 1, cu_h, _ptr(cu_dev), _tap_ptrs(taps), _tap_ld(taps),
        _ptr(w_c), _ptr(ctx_norm), _ptr(block_in), _ptr(block_pos), arr, _ptr(out_norm),
        _ptr(h_ctx_out), _ptr(block_out), _ptr(ws), nbytes, ts.cuda_stream))
    return block_out


def cache_bytes(dims: DsparkDims, A: int, cap: int) -> int:
    dm = dims.c()
    n = L.lib().dspark_cache_bytes(ctypes.byref(dm), A, cap)
    if n == 0:
        raise DsparkError(L.EINVAL, L.lib().dspark_last_error().decode(errors="replace"))
    return int(n)


class DraftCache:
    """A draft cache (include/dspark.h, incremental context) for A sequences
    of up to ``cap`` context rows each: the device buffer, cleared on
    creation, and the sequences' lengths kept on the host. ``append`` runs
    dspark_ctx_append (Eq 2 + every layer's context K/V of the new rows into
    the cache), ``propose`` runs dspark_block_propose (the draft block over
    the cached rows)."""

    def __init__(self, dims: DsparkDims, A: int, cap: int, device="cuda:0", stream=None):
        self.dims, self.A, self.cap = dims, A, cap
        self.device = torch.device(device)
        ts = _torch_stream(stream)
        with torch.cuda.stream(ts):
            self.buf = torch.empty(cache_bytes(dims, A, cap), dtype=torch.uint8, device=self.device)
        self.lengths = [0] * A
        self.reset(stream=stream)

    def reset(self, stream=None) -> None:
        dm = self.dims.c()
        L.check(L.lib().dspark_cache_reset(ctypes.byref(dm), self.A, self.cap, _ptr(self.buf),
                                           _stream(stream)))
        self.lengths = [0] * self.A

    def cu(self) -> List[int]:
        """Prefix offsets of the cached lengths."""
        out = [0]
        for n in self.lengths:
            out.append(out[-1] + n)
        return out

    def append(self, taps, counts: Sequence[int], w_c, ctx_norm, layers, *, ws=None,
               stream=None) -> None:
        """Append counts[b] new context rows to sequence b; the new rows of
        all sequences are packed in the taps in sequence order."""
        counts = [int(c) for c in counts]
        if len(counts) != self.A:
            raise ValueError(f"{len(counts)} counts for {self.A} sequences")
        ncu = [0]
        for c in counts:
            ncu.append(ncu[-1] + c)
        taps = _tap_list(taps, self.dims)
        ncu_h = _cu_host(ncu)
        pos_h = (ctypes.c_int32 * self.A)(*self.lengths)
        ts = _torch_stream(stream)
        with torch.cuda.stream(ts):
            ncu_d = torch.as_tensor(ncu, dtype=torch.int32, device=self.device)
            pos_d = torch.as_tensor(self.lengths, dtype=torch.int32, device=self.device)
            ws, nbytes = _workspace(L.OP_CTX_APPEND, self.dims, ncu, ws, self.device)
        dm = self.dims.c()
        arr = (L.LayerWeights * len(layers))(*[_layer_struct(lw) for lw in layers])
        L.check(L.lib().dspark_ctx_append(ctypes.byref(dm), self.A, self.cap, ncu_h, _ptr(ncu_d), pos_h,
                                          _ptr(pos_d), _tap_ptrs(taps), _tap_ld(taps), _ptr(w_c),
                                          _ptr(ctx_norm), arr, _ptr(self.buf), _ptr(ws), nbytes,
                                          ts.cuda_stream))
        self.lengths = [n + c for n, c in zip(self.lengths, counts)]

    def propose(self, block_in, block_pos, layers, out_norm=None, *, block_out=None, ws=None,
                cu_dev=None, stream=None) -> torch.Tensor:
        """The draft block [A, gamma, d] over the cached context."""
        cu = self.cu()
        cu_h = _cu_host(cu)
        ts = _torch_stream(stream)
        with torch.cuda.stream(ts):
            if block_out is None:
                block_out = torch.empty_like(block_in)
            cu_dev = _cu_dev(cu, cu_dev, self.device)
            ws, nbytes = _workspace(L.OP_BLOCK_PROPOSE, self.dims, cu, ws, self.device)
        dm = self.dims.c()
        arr = (L.LayerWeights * len(layers))(*[_layer_struct(lw) for lw in layers])
        L.check(L.lib().dspark_block_propose(ctypes.byref(dm), self.A, self.cap, cu_h, _ptr(cu_dev),
                                             _ptr(self.buf), _ptr(block_in), _ptr(block_pos), arr,
                                             _ptr(out_norm), _ptr(block_out), _ptr(ws), nbytes,
                                             ts.cuda_stream))
        return block_out


def block_build(dims: DsparkDims, anchor_emb, tok_proj, mask_emb, *, block_in=None,
                stream=None) -> torch.Tensor:
    """#buildBlock's token rows [A, gamma, d] (float32, before block_pos):
    anchor_emb [A, H] float32, tok_proj [d, H] storage dtype, mask_emb
    [gamma-1, d] float32."""
    A = int(anchor_emb.shape[0])
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if block_in is None:
            block_in = torch.empty((A, dims.gamma, dims.d), dtype=torch.float32, device=anchor_emb.device)
    dm = dims.c()
    L.check(L.lib().dspark_block_build(ctypes.byref(dm), A, _ptr(anchor_emb), _ptr(tok_proj),
                                       _ptr(mask_emb), _ptr(block_in), ts.cuda_stream))
    return block_in


def padded_workspace_size(dims: DsparkDims, A: int, L_ctx: int) -> int:
    """Workspace bytes of block_forward_padded (dspark_padded_workspace_size)."""
    dm = dims.c()
    n = L.lib().dspark_padded_workspace_size(ctypes.byref(dm), A, L_ctx)
    if n == 0:
        raise DsparkError(L.EINVAL, L.lib().dspark_last_error().decode(errors="replace"))
    return int(n)


def markov_workspace_size(dims: DsparkDims, A: int, vocab: int, rank: int) -> int:
    """Workspace bytes of markov_draft (dspark_markov_workspace_size)."""
    dm = dims.c()
    n = L.lib().dspark_markov_workspace_size(ctypes.byref(dm), A, vocab, rank)
    if n == 0:
        raise DsparkError(L.EINVAL, L.lib().dspark_last_error().decode(errors="replace"))
    return int(n)


def block_forward_padded(dims: DsparkDims, taps, L_ctx: int, ctx_mask, w_c, ctx_norm, block_in,
                         block_pos, layers, out_norm=None, *, h_ctx_out=None, block_out=None,
                         ws=None, stream=None) -> torch.Tensor:
    """The draft block of a padded batch: taps [A * L_ctx, H] per tap,
    ctx_mask [A, L_ctx] uint8 (1 = real row, 0 = padding)."""
    A = int(block_in.shape[0])
    taps = _tap_list(taps, dims)
    ts = _torch_stream(stream)
    dm = dims.c()
    with torch.cuda.stream(ts):
        if block_out is None:
            block_out = torch.empty_like(block_in)
        need = L.lib().dspark_padded_workspace_size(ctypes.byref(dm), A, L_ctx)
        if need == 0:
            raise DsparkError(L.EINVAL, L.lib().dspark_last_error().decode(errors="replace"))
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=block_in.device)
    arr = (L.LayerWeights * len(layers))(*[_layer_struct(lw) for lw in layers])
    L.check(L.lib().dspark_block_forward_padded(
        ctypes.byref(dm), A, L_ctx, _tap_ptrs(taps), _tap_ld(taps), _ptr(w_c), _ptr(ctx_norm),
        _ptr(ctx_mask), _ptr(block_in), _ptr(block_pos), arr, _ptr(out_norm), _ptr(h_ctx_out),
        _ptr(block_out), _ptr(ws), ws.numel() * ws.element_size(), ts.cuda_stream))
    return block_out


def markov_draft(dims: DsparkDims, block, base_logits, anchor, w1, w2, conf_w, conf_b, *,
                 tokens=None, conf=None, draft_logits=None, ws=None, stream=None):
    """The greedy draft loop after the backbone: (tokens [A, gamma] int32,
    confidences [A, gamma], draft logits [A, gamma, vocab]). w1 and w2 are
    [vocab, rank] in the storage dtype; anchor [A] int32 and conf_b [1] on
    the device."""
    A, G, _ = block.shape
    vocab, rank = int(w1.shape[0]), int(w1.shape[1])
    dm = dims.c()
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        if tokens is None:
            tokens = torch.empty((A, G), dtype=torch.int32, device=block.device)
        if conf is None:
            conf = torch.empty((A, G), dtype=torch.float32, device=block.device)
        if draft_logits is None:
            draft_logits = torch.empty((A, G, vocab), dtype=torch.float32, device=block.device)
        need = L.lib().dspark_markov_workspace_size(ctypes.byref(dm), A, vocab, rank)
        if need == 0:
            raise DsparkError(L.EINVAL, L.lib().dspark_last_error().decode(errors="replace"))
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device=block.device)
    L.check(L.lib().dspark_markov_draft(ctypes.byref(dm), A, vocab, rank, _ptr(block), _ptr(base_logits),
                                        _ptr(anchor), _ptr(w1), _ptr(w2), _ptr(conf_w), _ptr(conf_b),
                                        _ptr(tokens), _ptr(conf), _ptr(draft_logits), _ptr(ws),
                                        ws.numel() * ws.element_size(), ts.cuda_stream))
    return tokens, conf, draft_logits


class PreparedCall:
    """A library call with every argument marshalled once (outputs and
    workspace allocated up front); calling it only enqueues the call. Used
    to time the library without Python overhead. The tensors it was built
    from must stay alive while it is used."""

    def __init__(self, fn, args, keep, out=None):
        self.fn, self.args, self._keep, self.out = fn, args, keep, out

    def __call__(self):
        st = self.fn(*self.args)
        if st != L.OK:
            L.check(st)
        return self.out


def prepared_propose(cache: "DraftCache", block_in, block_pos, layers, out_norm=None, *,
                     stream=None) -> PreparedCall:
    """dspark_block_propose over the cache's current lengths, prepared."""
    cu = cache.cu()
    cu_h = _cu_host(cu)
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        out = torch.empty_like(block_in)
        cu_dev = _cu_dev(cu, None, cache.device)
        ws, nbytes = _workspace(L.OP_BLOCK_PROPOSE, cache.dims, cu, None, cache.device)
    dm = cache.dims.c()
    arr = (L.LayerWeights * len(layers))(*[_layer_struct(lw) for lw in layers])
    args = (ctypes.byref(dm), cache.A, cache.cap, cu_h, _ptr(cu_dev), _ptr(cache.buf), _ptr(block_in),
            _ptr(block_pos), arr, _ptr(out_norm), _ptr(out), _ptr(ws), nbytes, ts.cuda_stream)
    return PreparedCall(L.lib().dspark_block_propose, args,
                        (dm, cu_h, cu_dev, ws, arr, block_in, block_pos, layers, out_norm), out)


def prepared_append(cache: "DraftCache", taps, counts: Sequence[int], w_c, ctx_norm, layers, *,
                    stream=None) -> PreparedCall:
    """dspark_ctx_append of counts[b] rows at the cache's current lengths,
    prepared; repeated calls rewrite the same rows (the host lengths are
    not advanced), which is what a timing loop wants."""
    counts = [int(c) for c in counts]
    ncu = [0]
    for c in counts:
        ncu.append(ncu[-1] + c)
    taps = _tap_list(taps, cache.dims)
    ncu_h = _cu_host(ncu)
    pos_h = (ctypes.c_int32 * cache.A)(*cache.lengths)
    ts = _torch_stream(stream)
    with torch.cuda.stream(ts):
        ncu_d = torch.as_tensor(ncu, dtype=torch.int32, device=cache.device)
        pos_d = torch.as_tensor(cache.lengths, dtype=torch.int32, device=cache.device)
        ws, nbytes = _workspace(L.OP_CTX_APPEND, cache.dims, ncu, None, cache.device)
    dm = cache.dims.c()
    arr = (L.LayerWeights * len(layers))(*[_layer_struct(lw) for lw in layers])
    tp = _tap_ptrs(taps)
    args = (ctypes.byref(dm), cache.A, cache.cap, ncu_h, _ptr(ncu_d), pos_h, _ptr(pos_d), tp,
            _tap_ld(taps), _ptr(w_c), _ptr(ctx_norm), arr, _ptr(cache.buf), _ptr(ws), nbytes,
            ts.cuda_stream)
    return PreparedCall(L.lib().dspark_ctx_append, args,
                        (dm, ncu_h, pos_h, ncu_d, pos_d, ws, arr, tp, taps, w_c, ctx_norm, layers))


class PreparedForward:
    """block_forward with every argument marshalled once; calling it only
    enqueues the forward (used to time the library without Python overhead).
    The tensors passed in must stay alive while this object is used."""

    def __init__(self, dims: DsparkDims, cu, taps, w_c, ctx_norm, block_in, block_pos,
                 layers, out_norm=None, *, cu_dev=None, h_ctx_out=None, block_out=None,
                 ws=None, stream=None):
        device = block_in.device
        self.cu_h = _cu_host(cu)
        taps = _tap_list(taps, dims)
        ts = _torch_stream(stream)
        self.stream = ts
        with torch.cuda.stream(ts):
            self.block_out = torch.empty_like(block_in) if block_out is None else block_out
            self.cu_dev = _cu_dev(cu, cu_dev, device)
            self.ws, nbytes = _workspace(L.OP_BLOCK_FORWARD, dims, cu, ws, device)
        self.dm = dims.c()
        self.layers = (L.LayerWeights * len(layers))(*[_layer_struct(lw) for lw in layers])
        self.taps = _tap_ptrs(taps)
        self._keep = (taps, w_c, ctx_norm, block_in, block_pos, layers, out_norm, h_ctx_out)
        self.args = (ctypes.byref(self.dm), len(self.cu_h) - 1, self.cu_h, _ptr(self.cu_dev),
                     self.taps, _tap_ld(taps), _ptr(w_c), _ptr(ctx_norm), _ptr(block_in),
                     _ptr(block_pos), self.layers, _ptr(out_norm), _ptr(h_ctx_out),
                     _ptr(self.block_out), _ptr(self.ws), nbytes, ts.cuda_stream)
        self.fn = L.lib().dspark_block_forward

    def __call__(self) -> torch.Tensor:
        st = self.fn(*self.args)
        if st != L.OK:
            L.check(st)
        return self.block_out


def trace_begin(kinds: Sequence[str], capacity: int = 4096) -> None:
    """Record HIP events around every later launch of the named kernel kinds."""
    names = kernel_names()
    mask = 0
    for k in kinds:
        mask |= 1 << names.index(k)
    L.check(L.lib().dspark_trace_begin(mask, capacity))


def trace_end() -> Dict[str, tuple]:
    """Stop tracing; {kind: (total_ms, launches)} for kinds that launched."""
    names = kernel_names()
    n = len(names)
    tot = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    L.check(L.lib().dspark_trace_end(tot, cnt, n))
    return {names[i]: (tot[i], cnt[i]) for i in range(n) if cnt[i] > 0}
