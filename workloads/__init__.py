"""Seeded synthetic inputs for the draft-block forward (Eq 2 + Eq 3).

This module is shared by the CPU oracle, the tests and the benchmark. It
only *draws* numbers: it holds none of the method's arithmetic (no norm,
projection, attention or FFN). Every array is drawn in float32 from
``numpy.random.default_rng(SeedSequence([config_id, stream_id]))``, one
stream per tensor, then rounded to the storage precision of the workload
(bfloat16, round-to-nearest-even) so that the oracle and the GPU read the
exact same values.

Shapes, distributions and defaults follow the DFlash drafter on the page
"mlx-bun 0.0.7 -> 0.0.9, package/src/spec/dspark/module-dflash.ts"
(``DEFAULT_DFLASH_CONFIG`` and ``initFromDims``): weights are [in, out] and
applied as ``x @ W``; matrices ~ N(0, 0.02); norm gains start at 1. The
block rows follow ``#buildBlock``'s shape: row 0 stands for the anchor row
``anchor_emb @ tok_proj`` and is drawn directly from that product's
distribution, N(0, H * 0.02^2), rather than computed (this module holds no
arithmetic of the method; the product itself is ``dspark_block_build``,
whose inputs ``block_build_inputs`` draws); rows 1 .. gamma-1 are the shared
mask-embedding rows.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload", "make_inputs", "bf16_round",
    "bf16_bits", "small_workload",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic problem instance description."""

    name: str
    seed_id: int
    A: int                 # sequences in the packed batch
    m: int                 # tapped target layers
    H: int                 # target hidden width
    d: int                 # draft width (dDraft)
    n_heads: int
    gamma: int             # block size
    n_layers: int          # draft layers
    ff: int                # FFN width (ffMult * d)
    dtype: str             # "f32" or "bf16": storage precision of long tensors
    L: Optional[int] = None            # context length (all sequences), or
    L_range: Optional[tuple] = None    # (lo, hi) inclusive for ragged batches
    outlier_frac: float = 0.0          # fraction of context rows scaled x8
    outlier_scale: float = 8.0
    eps: float = 1e-6

    @property
    def head_dim(self) -> int:
        return self.d // self.n_heads


# The five problem instances. Sizes follow the drafter defaults on the
# module-dflash.ts page (gamma=5, dDraft=1024, nLayers=5, nHeads=8, ffMult=2,
# four tapped layers) and the five-tap layout of the dspark-runtime.js page
# (DSPARK_LAYERS has five entries).
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny-f32-L64", 1, A=1, m=4, H=256, d=128, n_heads=4, gamma=5,
                 n_layers=1, ff=256, dtype="f32", L=64),
        Workload("bf16-L2048-d1024", 2, A=1, m=4, H=2560, d=1024, n_heads=8,
                 gamma=5, n_layers=5, ff=2048, dtype="bf16", L=2048),
        Workload("bf16-L8192-d2048-outliers", 3, A=1, m=5, H=2048, d=2048,
                 n_heads=16, gamma=8, n_layers=5, ff=4096, dtype="bf16",
                 L=8192, outlier_frac=0.01),
        Workload("bf16-ragged16-L512..16384", 4, A=16, m=4, H=2560, d=1024,
                 n_heads=8, gamma=5, n_layers=5, ff=2048, dtype="bf16",
                 L_range=(512, 16384)),
        Workload("bf16-L131072", 5, A=1, m=4, H=2560, d=1024, n_heads=8,
                 gamma=5, n_layers=5, ff=2048, dtype="bf16", L=131072),
    ]
}


def get_workload(name: str) -> Workload:
    if name in WORKLOADS:
        return WORKLOADS[name]
    raise KeyError(f"unknown workload {name!r}; known: {sorted(WORKLOADS)}")


def small_workload(name="small", *, A=1, m=2, H=64, d=64, n_heads=2, gamma=3,
                   n_layers=1, ff=None, dtype="bf16", L=None, L_range=None,
                   lengths=None, seed_id=100, outlier_frac=0.0, eps=1e-6) -> Workload:
    """A custom (usually small) workload for tests."""
    if ff is None:
        ff = 2 * d
    if L is None and L_range is None:
        L = 16
    w = Workload(name, seed_id, A=A, m=m, H=H, d=d, n_heads=n_heads,
                 gamma=gamma, n_layers=n_layers, ff=ff, dtype=dtype, L=L,
                 L_range=L_range, outlier_frac=outlier_frac, eps=eps)
    return w


# ----------------------------------------------------------------------------
# bfloat16 storage helpers (a storage format, not part of the method)
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    NaN/Inf do not occur in these workloads.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (RNE); returns float32."""
    b = bf16_bits(x).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def _rng(seed_id: int, stream: int, variant: int = 0, chunk: int = 0) -> np.random.Generator:
    return np.random.default_rng(
        np.random.SeedSequence([seed_id, stream, variant, chunk]))


_CHUNK_ROWS = 512
_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures
        import os
        n = max(1, min(16, len(os.sched_getaffinity(0))))
        _POOL = concurrent.futures.ThreadPoolExecutor(max_workers=n)
    return _POOL


def _normal(seed_id, stream, shape, std, variant=0, round_bf16=False):
    """float32 N(0, std^2) draws.

    Arrays are drawn in blocks of ``_CHUNK_ROWS`` leading-axis rows, each from
    its own stream ``[seed_id, stream, variant, block]``, so the values do not
    depend on how many threads fill them.
    """
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float32)
    rows = shape[0] if shape else 1
    nblk = max(1, -(-rows // _CHUNK_ROWS))

    def fill(c):
        r0, r1 = c * _CHUNK_ROWS, min(rows, (c + 1) * _CHUNK_ROWS)
        view = out[r0:r1] if shape else out
        _rng(seed_id, stream, variant, c).standard_normal(
            view.shape, dtype=np.float32, out=view)
        if std != 1.0:
            view *= np.float32(std)
        if round_bf16:
            view[...] = bf16_round(view)

    if nblk == 1:
        fill(0)
    else:
        list(_pool().map(fill, range(nblk)))
    return out


# Stream ids: taps 0..m-1, then fixed ids for the rest (kept stable so adding a
# tensor never shifts the others).
_S_WC, _S_LAYER0, _S_PER_LAYER = 20, 100, 10
_S_ANCHOR, _S_MASK, _S_POS, _S_LEN, _S_OUTL = 40, 42, 43, 44, 45
_S_GAINS = 60


def context_lengths(w: Workload, lengths: Optional[List[int]] = None) -> np.ndarray:
    """Per-sequence context lengths L_b (int64)."""
    if lengths is not None:
        Ls = np.asarray(lengths, dtype=np.int64)
        assert Ls.shape == (w.A,)
        return Ls
    if w.L_range is not None:
        lo, hi = w.L_range
        return _rng(w.seed_id, _S_LEN).integers(lo, hi, size=w.A, endpoint=True).astype(np.int64)
    return np.full(w.A, int(w.L), dtype=np.int64)


def make_inputs(w: Workload, *, gains: str = "unit", lengths=None,
                with_taps: bool = True) -> dict:
    """Draw every input of one forward.

    Returns a dict of float32 numpy arrays whose values are exactly
    representable in the workload's storage precision:

    ``taps``       list of m arrays [T, H] (context rows of all sequences packed)
    ``cu``         int64 [A+1] prefix offsets of the packed context rows
    ``w_c``        [m*H, d]; ``ctx_norm`` [d]
    ``layers``     list of dicts with attn_norm [d], wq/wk/wv/wo [d,d],
                   ff_norm [d], w_gate/w_up [d,ff], w_down [ff,d]
    ``block_in``   [A, gamma, d] float32 (anchor row, then mask rows)
    ``block_pos``  [gamma, d]; ``out_norm`` [d]

    ``gains="random"`` draws every norm gain from U(0.5, 1.5) instead of 1.
    """
    Ls = context_lengths(w, lengths)
    cu = np.zeros(w.A + 1, dtype=np.int64)
    cu[1:] = np.cumsum(Ls)
    T = int(cu[-1])

    out = {"cu": cu, "lengths": Ls, "T": T}
    if with_taps:
        n_out = int(round(w.outlier_frac * T))
        rows = None
        if n_out > 0:
            rows = np.sort(_rng(w.seed_id, _S_OUTL).choice(T, size=n_out, replace=False))
            out["outlier_rows"] = rows
        taps = []
        for j in range(w.m):
            t = _normal(w.seed_id, j, (T, w.H), 1.0,
                        round_bf16=(w.dtype == "bf16" and rows is None))
            if rows is not None:
                # outlier rows are scaled before rounding to the storage format
                t[rows] *= np.float32(w.outlier_scale)
                if w.dtype == "bf16":
                    blocks = range(0, T, _CHUNK_ROWS)
                    def rb(r0, t=t):
                        t[r0:r0 + _CHUNK_ROWS] = bf16_round(t[r0:r0 + _CHUNK_ROWS])
                    list(_pool().map(rb, blocks))
            taps.append(t)
        out["taps"] = taps

    def gain(stream):
        if gains == "unit":
            return np.ones(w.d, dtype=np.float32)
        g = _rng(w.seed_id, _S_GAINS + stream).uniform(0.5, 1.5, size=w.d)
        return g.astype(np.float32)

    bf = w.dtype == "bf16"
    out["w_c"] = _normal(w.seed_id, _S_WC, (w.m * w.H, w.d), 0.02, round_bf16=bf)
    out["ctx_norm"] = gain(0)
    layers = []
    for i in range(w.n_layers):
        s = _S_LAYER0 + _S_PER_LAYER * i
        lw = {
            "attn_norm": gain(1 + 2 * i),
            "wq": _normal(w.seed_id, s + 0, (w.d, w.d), 0.02, round_bf16=bf),
            "wk": _normal(w.seed_id, s + 1, (w.d, w.d), 0.02, round_bf16=bf),
            "wv": _normal(w.seed_id, s + 2, (w.d, w.d), 0.02, round_bf16=bf),
            "wo": _normal(w.seed_id, s + 3, (w.d, w.d), 0.02, round_bf16=bf),
            "ff_norm": gain(2 + 2 * i),
            "w_gate": _normal(w.seed_id, s + 4, (w.d, w.ff), 0.02, round_bf16=bf),
            "w_up": _normal(w.seed_id, s + 5, (w.d, w.ff), 0.02, round_bf16=bf),
            "w_down": _normal(w.seed_id, s + 6, (w.ff, w.d), 0.02, round_bf16=bf),
        }
        layers.append(lw)
    out["layers"] = layers
    out["out_norm"] = gain(99)

    # Block rows: row 0 stands for the anchor row anchor_emb @ tok_proj of
    # #buildBlock (anchor_emb ~ N(0,1) [H], tok_proj ~ N(0,0.02) [H,d]); each
    # of its entries is a sum of H such products, so it is drawn directly from
    # the same distribution N(0, H * 0.02^2). Rows 1..gamma-1 are the shared
    # mask embedding rows ~ N(0, 0.02). block_pos is kept separate and is
    # added by the forward.
    anchor_std = 0.02 * float(np.sqrt(w.H))
    anchor_row = _normal(w.seed_id, _S_ANCHOR, (w.A, w.d), anchor_std)
    mask_emb = _normal(w.seed_id, _S_MASK, (max(w.gamma - 1, 0), w.d), 0.02)
    block_in = np.empty((w.A, w.gamma, w.d), dtype=np.float32)
    block_in[:, 0, :] = anchor_row
    if w.gamma > 1:
        block_in[:, 1:, :] = mask_emb[None, :, :]
    out["block_in"] = block_in
    out["block_pos"] = _normal(w.seed_id, _S_POS, (w.gamma, w.d), 0.02)
    return out


# ----------------------------------------------------------------------------
# Markov head inputs (forwardInfer after the backbone)
# ----------------------------------------------------------------------------
_S_MK_BLOCK, _S_MK_U, _S_MK_ANCHOR, _S_MK_W1, _S_MK_W2, _S_MK_CW = 200, 201, 202, 203, 204, 205


def markov_inputs(seed_id: int, *, A: int, gamma: int, d: int, vocab: int, rank: int,
                  dtype: str = "bf16", u_std: float = 2.0, w1_std: float = 1.0,
                  w2_std: float = 0.1, zero_w2: bool = False) -> dict:
    """Seeded inputs of the greedy draft loop: the draft block [A, gamma, d]
    (N(0,1), the scale of normalised rows), base logits [A, gamma, vocab]
    ~ N(0, u_std^2), anchor tokens, w1 / w2 [vocab, rank] (w2 stored as
    [vocab, rank], i.e. the transpose of module-dflash.ts's [rank, vocab]),
    conf_w [d + rank] ~ N(0, 0.02^2), conf_b. w1 and w2 are rounded to the
    storage precision. initFromDims starts w2 at zero (``zero_w2``); the
    default scales make the Markov bias comparable to the base logits, so
    the previous token matters."""
    bf = dtype == "bf16"
    out = {
        "block": _normal(seed_id, _S_MK_BLOCK, (A, gamma, d), 1.0),
        "base_logits": _normal(seed_id, _S_MK_U, (A, gamma, vocab), u_std),
        "anchor": _rng(seed_id, _S_MK_ANCHOR).integers(0, vocab, size=A).astype(np.int32),
        "w1": _normal(seed_id, _S_MK_W1, (vocab, rank), w1_std, round_bf16=bf),
        "w2": (np.zeros((vocab, rank), dtype=np.float32) if zero_w2
               else _normal(seed_id, _S_MK_W2, (vocab, rank), w2_std, round_bf16=bf)),
        "conf_w": _normal(seed_id, _S_MK_CW, (d + rank,), 0.02),
        "conf_b": np.array([0.1], dtype=np.float32),
    }
    return out


# ----------------------------------------------------------------------------
# #buildBlock inputs and padded batches
# ----------------------------------------------------------------------------
_S_BB_ANCHOR, _S_BB_TOKPROJ, _S_BB_MASK, _S_PAD_NOISE, _S_PAD_POS = 210, 211, 212, 213, 214


def block_build_inputs(seed_id: int, *, A: int, H: int, d: int, gamma: int, dtype: str = "bf16") -> dict:
    """anchor_emb [A, H] ~ N(0, 1) (an embedding row of the target), tok_proj
    [H, d] ~ N(0, 0.02^2) rounded to the storage precision, mask_emb
    [gamma-1, d] ~ N(0, 0.02^2) (initFromDims's distributions)."""
    return {
        "anchor_emb": _normal(seed_id, _S_BB_ANCHOR, (A, H), 1.0),
        "tok_proj": _normal(seed_id, _S_BB_TOKPROJ, (H, d), 0.02, round_bf16=dtype == "bf16"),
        "mask_emb": _normal(seed_id, _S_BB_MASK, (max(gamma - 1, 0), d), 0.02),
    }


def padded_layout(seed_id: int, taps, cu, L_ctx: int, placements, dtype: str = "bf16"):
    """A padded batch holding packed context rows: sequence b's rows go to the
    positions of placements[b] ("lead": the first L_b rows, "scatter":
    seeded distinct positions, or an explicit index array) of its L_ctx slots;
    the other slots are padding filled with N(0, 3^2) noise. Returns the taps
    [A * L_ctx, H] and the mask [A, L_ctx] (uint8, 1 = real row)."""
    A = len(cu) - 1
    H = taps[0].shape[1]
    rng = _rng(seed_id, _S_PAD_POS)
    mask = np.zeros((A, L_ctx), dtype=np.uint8)
    out = [_normal(seed_id, _S_PAD_NOISE + j, (A * L_ctx, H), 3.0, round_bf16=dtype == "bf16")
           for j in range(len(taps))]
    for b in range(A):
        L = int(cu[b + 1] - cu[b])
        pl = placements[b]
        if isinstance(pl, str) and pl == "lead":
            pos = np.arange(L)
        elif isinstance(pl, str) and pl == "scatter":
            pos = np.sort(rng.choice(L_ctx, size=L, replace=False))
        else:
            pos = np.asarray(pl)
            assert len(pos) == L
        mask[b, pos] = 1
        for j, t in enumerate(taps):
            out[j][b * L_ctx + pos] = t[cu[b]:cu[b + 1]]
    return out, mask


# ----------------------------------------------------------------------------
# The page-1 layer variant: grouped K/V heads and q/k-norm gains
# ----------------------------------------------------------------------------
_S_VAR = 300


def variant_layers(w: Workload, layers: List[dict], n_kv_heads: int, *, gains: str = "random") -> List[dict]:
    """Copies of the layers for the variant: W_K, W_V redrawn as [d, n_kv * hd]
    when the K/V heads are grouped (N(0, 0.02^2), storage-rounded), and
    per-head q_norm / k_norm gains [hd] (U(0.5, 1.5), or 1 with
    gains="unit")."""
    hd = w.head_dim
    kvd = n_kv_heads * hd
    bf = w.dtype == "bf16"
    out = []
    for i, lw in enumerate(layers):
        v = dict(lw)
        s = _S_VAR + 10 * i
        if kvd != w.d:
            v["wk"] = _normal(w.seed_id, s + 0, (w.d, kvd), 0.02, round_bf16=bf)
            v["wv"] = _normal(w.seed_id, s + 1, (w.d, kvd), 0.02, round_bf16=bf)
        if gains == "unit":
            v["q_norm"] = np.ones(hd, dtype=np.float32)
            v["k_norm"] = np.ones(hd, dtype=np.float32)
        else:
            v["q_norm"] = _rng(w.seed_id, s + 2).uniform(0.5, 1.5, size=hd).astype(np.float32)
            v["k_norm"] = _rng(w.seed_id, s + 3).uniform(0.5, 1.5, size=hd).astype(np.float32)
        out.append(v)
    return out
