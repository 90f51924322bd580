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

Beyond the draft block itself the module holds, each in its own section:
  * the incremental context of "src/dspark-runtime.js" (``updateContext``,
    ``store``, ``propose``): a per-layer key/value cache filled by appends,
    and the block side over it;
  * the Markov head, confidence head and greedy draft loop of
    ``forwardInfer`` in module-dflash.ts (argmax ties go to the lowest
    index, numpy's rule);
  * ``#buildBlock`` and the padded-batch attention bias of ``#maskBias``;
  * the layer variant of "src/dspark-runtime.js": q/k norms with RoPE,
    fewer K/V heads than query heads, context rows projected without a
    per-layer norm. Readings where the page is silent: the norms are RMSNorms
    over one head with an [hd] gain; RoPE rotates the pair (c, c + hd/2) by
    pos * theta^(-2c/hd); context row t of a sequence sits at position t and
    block row j at L_b + j; query head h reads K/V head h // (n / n_kv).

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
    # incremental context (dspark-runtime.js updateContext / store / propose)
    "DraftCache", "cache_append", "propose_layer", "block_propose",
    # Markov head, confidence head, greedy loop (module-dflash.ts forwardInfer)
    "sigmoid", "markov_draft",
    # block construction and the padded-batch mask (#buildBlock, #maskBias)
    "build_block", "mask_bias", "attention_biased", "block_forward_padded",
    # page-1 layer variant (q/k norms, RoPE, grouped K/V heads, no context norm)
    "rope", "head_rmsnorm", "variant_context_kv", "variant_layer", "variant_forward",
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


# ============================================================================
# Incremental (cached) context: the page "src/dspark-runtime.js".
#
# Its updateContext(position, count) projects `count` new context rows (Eq 2:
# projectBatch/projectBlock, then the hidden norm), and for every draft layer
# projects them with that layer's K/V weights (contextBatch/contextBlock) and
# appends them to the layer's key/value cache (store). propose() then runs the
# block side of every layer over the cached keys and values. The context rows
# here follow module-dflash.ts (#layer normalises them with the layer's
# attention-norm gain before W_K / W_V), so a cache filled piece by piece
# holds exactly the K_c / V_c that #layer computes from the whole context.
# ============================================================================

class DraftCache:
    """Per-sequence, per-layer context keys and values (lists of [L_b, d])."""

    def __init__(self, A: int, n_layers: int, d: int, dtype=np.float64):
        self.dtype = dtype
        self.K = [[np.zeros((0, d), dtype=dtype) for _ in range(n_layers)] for _ in range(A)]
        self.V = [[np.zeros((0, d), dtype=dtype) for _ in range(n_layers)] for _ in range(A)]

    def lengths(self) -> np.ndarray:
        return np.array([k[0].shape[0] for k in self.K], dtype=np.int64)

    def packed(self, layer: int):
        """(K_c, V_c, cu) of one layer with the sequences packed."""
        Ls = self.lengths()
        cu = np.zeros(len(Ls) + 1, dtype=np.int64)
        cu[1:] = np.cumsum(Ls)
        Kc = np.concatenate([k[layer] for k in self.K], axis=0)
        Vc = np.concatenate([v[layer] for v in self.V], axis=0)
        return Kc, Vc, cu


def cache_append(cache: DraftCache, taps_new: Sequence[np.ndarray], cu_new: Sequence[int],
                 w_c: np.ndarray, ctx_norm: np.ndarray, layers: List[Dict[str, np.ndarray]],
                 eps: float) -> np.ndarray:
    """updateContext for every sequence: the new rows of sequence b are rows
    cu_new[b] .. cu_new[b+1]-1 of ``taps_new``; Eq 2 gives their context rows
    C, and each layer's K_c = RMSNorm(C; attn_norm) W_K, V_c = ... W_V rows are
    appended to that sequence's cache. Returns the new rows of C."""
    dt = cache.dtype
    f = lambda a: np.asarray(a, dtype=dt)
    C = ctx_fuse(taps_new, w_c, ctx_norm, eps, dtype=dt)
    for i, lw in enumerate(layers):
        Uc = rmsnorm(C, f(lw["attn_norm"]), eps)
        Kc, Vc = Uc @ f(lw["wk"]), Uc @ f(lw["wv"])
        for b in range(len(cache.K)):
            r0, r1 = int(cu_new[b]), int(cu_new[b + 1])
            cache.K[b][i] = np.concatenate([cache.K[b][i], Kc[r0:r1]], axis=0)
            cache.V[b][i] = np.concatenate([cache.V[b][i], Vc[r0:r1]], axis=0)
    return C


def propose_layer(Kc: np.ndarray, Vc: np.ndarray, cu: Sequence[int], D: np.ndarray,
                  lw: Dict[str, np.ndarray], n_heads: int, eps: float, dtype=np.float64,
                  act: str = "silu") -> np.ndarray:
    """One draft layer of propose(): the block rows D attend over the cached
    context keys/values of their sequence followed by their own keys (the
    rest of #layer unchanged)."""
    f = lambda a: np.asarray(a, dtype=dtype)
    D = f(D)
    U = rmsnorm(D, f(lw["attn_norm"]), eps)
    Q = U @ f(lw["wq"])
    Kd, Vd = U @ f(lw["wk"]), U @ f(lw["wv"])
    Attn = attention(Q, f(Kc), f(Vc), Kd, Vd, cu, n_heads)
    E = D + Attn @ f(lw["wo"])
    Z = rmsnorm(E, f(lw["ff_norm"]), eps)
    a = silu(Z @ f(lw["w_gate"])) if act == "silu" else gelu_tanh(Z @ f(lw["w_gate"]))
    return E + (a * (Z @ f(lw["w_up"]))) @ f(lw["w_down"])


def block_propose(cache: DraftCache, block_in: np.ndarray, block_pos: np.ndarray,
                  layers: List[Dict[str, np.ndarray]], out_norm: Optional[np.ndarray],
                  n_heads: int, eps: float) -> np.ndarray:
    """propose(): block init, every layer over its cached context, output norm."""
    dt = cache.dtype
    D = block_init(block_in, block_pos, dtype=dt)
    for i, lw in enumerate(layers):
        Kc, Vc, cu = cache.packed(i)
        D = propose_layer(Kc, Vc, cu, D, lw, n_heads, eps, dtype=dt)
    return D if out_norm is None else rmsnorm(D, np.asarray(out_norm, dtype=dt), eps)


# ============================================================================
# Markov head, confidence head and the greedy draft loop: module-dflash.ts
# (#markov, #confidence, forwardInfer); the page "src/dspark-runtime.js" runs
# the same steps as markovEmbed -> markov -> addBias -> argmax per position.
# The base logits come from the target model's LM head (not computed here:
# they are an input).
# ============================================================================

def sigmoid(x: np.ndarray) -> np.ndarray:
    one = x.dtype.type(1.0)
    return one / (one + np.exp(-x))


def markov_draft(block: np.ndarray, base_logits: np.ndarray, anchor_tok: Sequence[int],
                 w1: np.ndarray, w2: np.ndarray, conf_w: np.ndarray, conf_b: float,
                 dtype=np.float64):
    """Greedy forwardInfer after the backbone, for every sequence b:
    prev = anchor token; for k < gamma: e1 = w1[prev] (the Markov embedding of
    the previous token), logits_k = base_logits[b, k] + e1 @ w2, token_k =
    argmax logits_k (the lowest index among equal maxima, numpy's rule),
    conf_k = sigmoid([block[b, k], e1] . conf_w + conf_b), prev = token_k.

    block [A, gamma, d] (the normalised backbone output), base_logits
    [A, gamma, V], w1 [V, r], w2 [r, V], conf_w [d + r]. Returns tokens
    [A, gamma] (int64), conf [A, gamma] and the draft logits [A, gamma, V]."""
    f = lambda a: np.asarray(a, dtype=dtype)
    block, U, w1, w2, cw = f(block), f(base_logits), f(w1), f(w2), f(conf_w).reshape(-1)
    A, G, _ = block.shape
    V = U.shape[-1]
    toks = np.zeros((A, G), dtype=np.int64)
    conf = np.zeros((A, G), dtype=dtype)
    logits = np.zeros((A, G, V), dtype=dtype)
    for b in range(A):
        prev = int(anchor_tok[b])
        for k in range(G):
            e1 = w1[prev]
            lk = U[b, k] + e1 @ w2
            tok = int(np.argmax(lk))
            conf[b, k] = sigmoid(np.concatenate([block[b, k], e1]) @ cw + dtype(conf_b))
            logits[b, k] = lk
            toks[b, k] = tok
            prev = tok
    return toks, conf, logits


# ============================================================================
# Block construction and the padded-batch attention mask: module-dflash.ts
# (#buildBlock, #maskBias, and #backbone / #layer with a mask).
# ============================================================================

def build_block(anchor_emb: np.ndarray, tok_proj: np.ndarray, mask_emb: np.ndarray,
                block_pos: np.ndarray, dtype=np.float64) -> np.ndarray:
    """#buildBlock: row 0 of each sequence is anchor_emb[b] @ tok_proj +
    block_pos[0]; rows 1 .. gamma-1 are mask_emb[j-1] + block_pos[j], the same
    for every sequence. anchor_emb [A, H], tok_proj [H, d], mask_emb
    [gamma-1, d], block_pos [gamma, d] -> H_d [A, gamma, d]."""
    f = lambda a: np.asarray(a, dtype=dtype)
    anchor = f(anchor_emb) @ f(tok_proj)
    bp = f(block_pos)
    A, G = anchor.shape[0], bp.shape[0]
    Hd = np.empty((A, G, bp.shape[1]), dtype=dtype)
    Hd[:, 0] = anchor + bp[0]
    if G > 1:
        Hd[:, 1:] = (f(mask_emb) + bp[1:])[None]
    return Hd


NEG = -1e9   # the padding bias of #maskBias


def mask_bias(ctx_mask: np.ndarray, gamma: int, dtype=np.float64) -> np.ndarray:
    """#maskBias: ctx_mask [A, Lctx] (1 = real row, 0 = padding) -> additive
    bias [A, Lctx + gamma]: (mask - 1) * 1e9 on the context columns (0 for
    real rows, -1e9 for padding) and 0 on the gamma block columns."""
    m = np.asarray(ctx_mask, dtype=dtype)
    ctx = (m - dtype(1.0)) * dtype(-NEG)
    return np.concatenate([ctx, np.zeros((m.shape[0], gamma), dtype=dtype)], axis=1)


def attention_biased(Q: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, Kd: np.ndarray,
                     Vd: np.ndarray, bias: np.ndarray, n_heads: int) -> np.ndarray:
    """sdpa of #layer on a padded batch: Q, Kd, Vd [A, gamma, d]; Kc, Vc
    [A, Lctx, d]; bias [A, Lctx + gamma] added to every head's scores."""
    A, gamma, d = Q.shape
    hd = d // n_heads
    scale = Q.dtype.type(1.0 / math.sqrt(hd))
    out = np.empty_like(Q)
    for b in range(A):
        for h in range(n_heads):
            cs = slice(h * hd, (h + 1) * hd)
            k = np.concatenate([Kc[b, :, cs], Kd[b, :, cs]], axis=0)
            v = np.concatenate([Vc[b, :, cs], Vd[b, :, cs]], axis=0)
            p = softmax((Q[b, :, cs] @ k.T) * scale + bias[b][None, :])
            out[b, :, cs] = p @ v
    return out


def block_forward_padded(taps: Sequence[np.ndarray], w_c: np.ndarray, ctx_norm: np.ndarray,
                         ctx_mask: np.ndarray, block_in: np.ndarray, block_pos: np.ndarray,
                         layers: List[Dict[str, np.ndarray]], out_norm: Optional[np.ndarray],
                         n_heads: int, eps: float, dtype=np.float64) -> np.ndarray:
    """#backbone on a padded batch: taps are [A, Lctx, H] (padding rows hold
    any finite values), ctx_mask [A, Lctx]; the -1e9 bias of #maskBias
    removes the padding rows from every softmax."""
    f = lambda a: np.asarray(a, dtype=dtype)
    A, Lctx = np.asarray(ctx_mask).shape
    X = np.concatenate([f(t) for t in taps], axis=2)            # [A, Lctx, m*H]
    C = rmsnorm(X @ f(w_c), f(ctx_norm), eps)                   # Eq 2 per row
    bias = mask_bias(ctx_mask, np.asarray(block_in).shape[1], dtype=dtype)
    D = block_init(block_in, block_pos, dtype=dtype)
    for lw in layers:
        g = f(lw["attn_norm"])
        U, Uc = rmsnorm(D, g, eps), rmsnorm(C, g, eps)
        Q = U @ f(lw["wq"])
        Kd, Vd = U @ f(lw["wk"]), U @ f(lw["wv"])
        Kc, Vc = Uc @ f(lw["wk"]), Uc @ f(lw["wv"])
        E = D + attention_biased(Q, Kc, Vc, Kd, Vd, bias, n_heads) @ f(lw["wo"])
        Z = rmsnorm(E, f(lw["ff_norm"]), eps)
        D = E + (silu(Z @ f(lw["w_gate"])) * (Z @ f(lw["w_up"]))) @ f(lw["w_down"])
    return D if out_norm is None else rmsnorm(D, f(out_norm), eps)


# ============================================================================
# The layer variant of the page "src/dspark-runtime.js": per layer q_norm and
# k_norm weights with rotary positions (its noiseNormRope / contextNormRope
# kernels), fewer key/value heads than query heads (its grids of 16 + 2
# heads), and context rows that enter W_K / W_V without a per-layer norm (its
# contextKV kernel reads the context directly). module-dflash.ts has none of
# these; with all of them switched off the variant is #layer exactly.
#
# Readings (the page prints no formula): q_norm / k_norm are RMSNorms over
# one head's hd values with an [hd] gain; RoPE rotates the pair (c, c + hd/2)
# of a head by the angle pos * theta^(-2c/hd); a context row's position is
# its index in its sequence, block row j's is L_b + j; query head h reads
# key/value head h // (n_heads / n_kv_heads).
# ============================================================================

def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding of x [..., rows, hd] at integer positions pos [rows]:
    (x_c, x_{c+hd/2}) -> (x_c cos a - x_{c+hd/2} sin a, x_{c+hd/2} cos a + x_c sin a)
    with a = pos * theta^(-2c/hd), c < hd/2."""
    hd = x.shape[-1]
    half = hd // 2
    inv = np.asarray(theta, dtype=np.float64) ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]    # [rows, hd/2]
    c, s = np.cos(ang).astype(x.dtype), np.sin(ang).astype(x.dtype)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def head_rmsnorm(x: np.ndarray, g: np.ndarray, n_heads: int, eps: float) -> np.ndarray:
    """RMSNorm over each head's hd values of x [..., n_heads * hd], gain g [hd]."""
    hd = x.shape[-1] // n_heads
    xs = x.reshape(x.shape[:-1] + (n_heads, hd))
    return rmsnorm(xs, np.asarray(g, dtype=x.dtype), eps).reshape(x.shape)


def _positions_rows(x: np.ndarray, n_heads: int, pos: np.ndarray, theta: float) -> np.ndarray:
    """RoPE on every head of x [rows, n_heads * hd] at positions pos [rows]."""
    hd = x.shape[-1] // n_heads
    xs = x.reshape(x.shape[0], n_heads, hd).transpose(1, 0, 2)   # [heads, rows, hd]
    return rope(xs, pos, theta).transpose(1, 0, 2).reshape(x.shape)


def variant_context_kv(C: np.ndarray, cu: Sequence[int], lw: Dict[str, np.ndarray],
                       n_kv_heads: int, eps: float, *, ctx_norm_kv: bool, qk_norm: bool,
                       theta: float, dtype=np.float64):
    """The context keys/values of one layer: [RMSNorm(C; attn_norm)] W_K, W_V,
    then k_norm and RoPE on the keys at each row's position in its sequence."""
    f = lambda a: np.asarray(a, dtype=dtype)
    C = f(C)
    X = rmsnorm(C, f(lw["attn_norm"]), eps) if ctx_norm_kv else C
    Kc, Vc = X @ f(lw["wk"]), X @ f(lw["wv"])
    if qk_norm:
        Kc = head_rmsnorm(Kc, lw["k_norm"], n_kv_heads, eps)
    if theta > 0:
        pos = np.concatenate([np.arange(int(cu[b + 1]) - int(cu[b])) for b in range(len(cu) - 1)])
        Kc = _positions_rows(Kc, n_kv_heads, pos.astype(np.int64), theta)
    return Kc, Vc


def variant_layer(Kc: np.ndarray, Vc: np.ndarray, cu: Sequence[int], D: np.ndarray,
                  lw: Dict[str, np.ndarray], n_heads: int, n_kv_heads: int, eps: float, *,
                  qk_norm: bool, theta: float, act: str = "silu", dtype=np.float64) -> np.ndarray:
    """One variant layer on the block rows D [A, gamma, d] over the given
    context keys/values Kc, Vc [T, n_kv_heads * hd] (packed by cu)."""
    f = lambda a: np.asarray(a, dtype=dtype)
    D = f(D)
    A, G, d = D.shape
    hd = d // n_heads
    grp = n_heads // n_kv_heads
    U = rmsnorm(D, f(lw["attn_norm"]), eps)
    Q, Kd, Vd = U @ f(lw["wq"]), U @ f(lw["wk"]), U @ f(lw["wv"])
    if qk_norm:
        Q = head_rmsnorm(Q, lw["q_norm"], n_heads, eps)
        Kd = head_rmsnorm(Kd, lw["k_norm"], n_kv_heads, eps)
    Attn = np.empty_like(Q)
    scale = dtype(1.0 / math.sqrt(hd))
    for b in range(A):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        L = r1 - r0
        qb, kdb = Q[b], Kd[b]
        if theta > 0:
            bpos = np.arange(L, L + G, dtype=np.int64)
            qb = _positions_rows(qb, n_heads, bpos, theta)
            kdb = _positions_rows(kdb, n_kv_heads, bpos, theta)
        for h in range(n_heads):
            kh = h // grp
            qs, ks = slice(h * hd, (h + 1) * hd), slice(kh * hd, (kh + 1) * hd)
            k = np.concatenate([f(Kc)[r0:r1, ks], kdb[:, ks]], axis=0)
            v = np.concatenate([f(Vc)[r0:r1, ks], Vd[b][:, ks]], axis=0)
            p = softmax((qb[:, qs] @ k.T) * scale)
            Attn[b, :, qs] = p @ v
    E = D + Attn @ f(lw["wo"])
    Z = rmsnorm(E, f(lw["ff_norm"]), eps)
    g = Z @ f(lw["w_gate"])
    a = silu(g) if act == "silu" else gelu_tanh(g)
    return E + (a * (Z @ f(lw["w_up"]))) @ f(lw["w_down"])


def variant_forward(taps: Sequence[np.ndarray], w_c: np.ndarray, ctx_norm: np.ndarray,
                    cu: Sequence[int], block_in: np.ndarray, block_pos: np.ndarray,
                    layers: List[Dict[str, np.ndarray]], out_norm: Optional[np.ndarray],
                    n_heads: int, n_kv_heads: int, eps: float, *, ctx_norm_kv: bool = True,
                    qk_norm: bool = False, theta: float = 0.0, act: str = "silu",
                    dtype=np.float64) -> np.ndarray:
    """Eq 2, block init, every variant layer, output norm."""
    C = ctx_fuse(taps, w_c, ctx_norm, eps, dtype=dtype)
    D = block_init(block_in, block_pos, dtype=dtype)
    for lw in layers:
        Kc, Vc = variant_context_kv(C, cu, lw, n_kv_heads, eps, ctx_norm_kv=ctx_norm_kv,
                                    qk_norm=qk_norm, theta=theta, dtype=dtype)
        D = variant_layer(Kc, Vc, cu, D, lw, n_heads, n_kv_heads, eps, qk_norm=qk_norm,
                          theta=theta, act=act, dtype=dtype)
    return D if out_norm is None else rmsnorm(D, np.asarray(out_norm, dtype=dtype), eps)
