"""CPU oracle for the DSpark / DFlash draft-block forward (Eq 2 + Eq 3).

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module. It shares no code with
the HIP library and never imports it.

It is the plain definition of what the draft block computes, written from the
page "mlx-bun 0.0.7 -> 0.0.9, package/src/spec/dspark/module-dflash.ts" (the
header comment stating Eq 2 and Eq 3, and the ``#buildContext``,
``#buildBlock``, ``#layer`` and ``#backbone`` methods of ``DflashDrafter``)
and from the page "src/dspark-runtime.js" (the ``propose`` kernel order, which
fixes the gated FFN as SiLU(gate) * up). Numpy arrays, explicit per-sequence
and per-head loops, float64 by default (``dtype=np.float32`` gives the timed
single-precision mode). Nothing is blocked, fused or reordered.

Readings taken where the pages are silent or differ (each is listed in the
design notes of the repository):
  * RMSNorm(x; g) = x * (mean_k x_k^2 + eps)^(-1/2) * g  (multiplicative gain).
  * The FFN activation is SiLU(x) = x / (1 + exp(-x)) on the gate half
    (dspark-runtime.js runs a ``silu`` kernel between the fused gate/up and
    down projections); ``act="gelu_tanh"`` selects the tanh-GELU of
    module-dflash.ts instead.
  * The context rows are normalised with the layer's attention-norm gain
    before W_K / W_V, exactly as ``#layer`` does (same norm as the block).
  * Several sequences are packed along the context axis with prefix offsets
    ``cu``; sequence b attends to its own context rows only (the exact
    exclusion that the -1e9 key-padding bias of ``#maskBias`` produces).
  * There is no causal mask: the block attends bidirectionally.

Parity pins: every function below is checked in ``tests/test_oracle_pins.py``
against brute force, library routines, closed forms and invariants. The
exact rounding points of the bfloat16 GPU path are not modelled here
(parity unpinned for those roundings; they are covered by the tolerance).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np

__all__ = [
    "rmsnorm", "silu", "gelu_tanh", "ctx_fuse", "block_init", "softmax",
    "attention", "block_layer", "block_forward",
]


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """Row-wise RMSNorm with a multiplicative gain (``ops.rmsNorm`` in
    module-dflash.ts; gains are initialised to 1 in ``initFromDims``)."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + x.dtype.type(eps)) * g


def silu(x: np.ndarray) -> np.ndarray:
    """SiLU(x) = x * sigmoid(x) (the ``silu`` kernel of dspark-runtime.js)."""
    one = x.dtype.type(1.0)
    return x / (one + np.exp(-x))


def gelu_tanh(x: np.ndarray) -> np.ndarray:
    """tanh-approximated GELU (``ops.geluApprox`` in module-dflash.ts)."""
    c = x.dtype.type(math.sqrt(2.0 / math.pi))
    return x.dtype.type(0.5) * x * (x.dtype.type(1.0) + np.tanh(c * (x + x.dtype.type(0.044715) * x ** 3)))


def ctx_fuse(taps: Sequence[np.ndarray], w_c: np.ndarray, ctx_norm: np.ndarray,
             eps: float, dtype=np.float64) -> np.ndarray:
    """Eq 2: H_ctx = RMSNorm(W_c . [H^{l1}; ...; H^{lm}]).

    ``taps`` are the m tapped target hidden states [T, H]; they are
    concatenated on the feature axis in tap order (``#buildContext`` takes
    hCtx [A, Lctx, m*H]), projected by W_c [m*H, d] and normalised with the
    ``ctx_norm`` gain.
    """
    X = np.concatenate([np.asarray(t, dtype=dtype) for t in taps], axis=1)
    P = X @ np.asarray(w_c, dtype=dtype)
    return rmsnorm(P, np.asarray(ctx_norm, dtype=dtype), eps)


def block_init(block_in: np.ndarray, block_pos: np.ndarray, dtype=np.float64) -> np.ndarray:
    """Block rows before layer 0: token rows plus the learned block position
    (``#buildBlock`` adds ``block_pos[j]`` to block row j)."""
    return np.asarray(block_in, dtype=dtype) + np.asarray(block_pos, dtype=dtype)[None, :, :]


def softmax(s: np.ndarray) -> np.ndarray:
    """softmax over the last axis, exp(s - max) / sum exp(s - max)."""
    z = s - np.max(s, axis=-1, keepdims=True)
    e = np.exp(z)
    return e / np.sum(e, axis=-1, keepdims=True)


def attention(Q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, Kd: np.ndarray,
              Vd: np.ndarray, cu: Sequence[int], n_heads: int) -> np.ndarray:
    """Block attention of Eq 3 over [context ++ block].

    Q, Kd, Vd: [A, gamma, d] (block rows); Kc, Vc: [T, d] packed context
    rows, sequence b owning rows cu[b] .. cu[b+1]-1. For each sequence and
    head, the gamma queries attend over that sequence's context keys followed
    by its gamma block keys with weights softmax(q k^T * hd^-1/2) and no
    causal mask (``ops.sdpa`` with scale hd^-0.5 in ``#layer``). Heads are
    concatenated back to [A, gamma, d].
    """
    A, gamma, d = Q.shape
    hd = d // n_heads
    scale = Q.dtype.type(1.0 / math.sqrt(hd))
    out = np.empty_like(Q)
    for b in range(A):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        for h in range(n_heads):
            cs = slice(h * hd, (h + 1) * hd)
            q = Q[b, :, cs]                                      # [gamma, hd]
            k = np.concatenate([Kc[r0:r1, cs], Kd[b, :, cs]], axis=0)  # [L+gamma, hd]
            v = np.concatenate([Vc[r0:r1, cs], Vd[b, :, cs]], axis=0)
            p = softmax((q @ k.T) * scale)                       # [gamma, L+gamma]
            out[b, :, cs] = p @ v
    return out


def block_layer(C: np.ndarray, cu: Sequence[int], D: np.ndarray, lw: Dict[str, np.ndarray],
                n_heads: int, eps: float, dtype=np.float64, act: str = "silu",
                intermediates: Optional[dict] = None) -> np.ndarray:
    """Eq 3 plus the block FFN for one draft layer (``#layer``).

    C [T, d] is the read-only context memory (never modified); D [A, gamma, d]
    are the block rows. Returns the new block rows.
    """
    f = lambda a: np.asarray(a, dtype=dtype)
    C = f(C)
    D = f(D)
    g_a = f(lw["attn_norm"])
    U = rmsnorm(D, g_a, eps)          # block rows, attention norm
    Uc = rmsnorm(C, g_a, eps)         # context rows, the same norm and gain
    wk, wv = f(lw["wk"]), f(lw["wv"])
    Q = U @ f(lw["wq"])               # queries from the block only
    Kd, Vd = U @ wk, U @ wv           # block keys / values
    Kc, Vc = Uc @ wk, Uc @ wv         # context re-projected with this layer's W_K / W_V
    Attn = attention(Q, Kc, Vc, Kd, Vd, cu, n_heads)
    E = D + Attn @ f(lw["wo"])        # residual
    Z = rmsnorm(E, f(lw["ff_norm"]), eps)
    G = Z @ f(lw["w_gate"])
    Up = Z @ f(lw["w_up"])
    a = silu(G) if act == "silu" else gelu_tanh(G)
    out = E + (a * Up) @ f(lw["w_down"])   # residual
    if intermediates is not None:
        intermediates.update(dict(U=U, Q=Q, Kd=Kd, Vd=Vd, Kc=Kc, Vc=Vc,
                                  Attn=Attn, E=E, Z=Z, out=out))
    return out


def block_forward(taps: Sequence[np.ndarray], w_c: np.ndarray, ctx_norm: np.ndarray,
                  cu: Sequence[int], block_in: np.ndarray, block_pos: np.ndarray,
                  layers: List[Dict[str, np.ndarray]], out_norm: Optional[np.ndarray],
                  n_heads: int, eps: float, dtype=np.float64, act: str = "silu",
                  trace: Optional[dict] = None) -> np.ndarray:
    """``#backbone``: Eq 2, block init, every draft layer, output norm.

    Returns the normalised block rows [A, gamma, d] (or the un-normalised
    rows when ``out_norm`` is None). ``trace``, when given, receives the
    context memory ``C`` and the block rows after each layer (``D`` list).
    """
    C = ctx_fuse(taps, w_c, ctx_norm, eps, dtype=dtype)
    D = block_init(block_in, block_pos, dtype=dtype)
    Ds = [D]
    for lw in layers:
        D = block_layer(C, cu, D, lw, n_heads, eps, dtype=dtype, act=act)
        Ds.append(D)
    out = D if out_norm is None else rmsnorm(D, np.asarray(out_norm, dtype=dtype), eps)
    if trace is not None:
        trace["C"] = C
        trace["D"] = Ds
        trace["out"] = out
    return out
