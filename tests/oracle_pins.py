"""Checks that pin the CPU oracle to things other than itself.

Each ``pin_*`` function takes the oracle module and raises AssertionError when
the oracle disagrees with an independent fact: a brute-force scalar
implementation, a library routine (torch), a closed form or an invariant of
the method stated on the pages (module-dflash.ts header comment: context is
read-only memory re-projected at every layer, the block attends
bidirectionally over [context ++ block]). ``tests/test_oracle_mutations.py``
plants mistakes in the oracle and checks that at least one pin fails.
"""
from __future__ import annotations

import hashlib
import math

import numpy as np

TIGHT = 1e-11


def rel_err(y, r):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    return float(np.max(np.abs(y - r)) / max(np.max(np.abs(r)), 1e-300))


def _rand_problem(rs, *, lengths, m=2, H=3, d=4, n_heads=2, gamma=3, n_layers=2,
                  ff=6, gains_random=True, w_std=0.5):
    """Small random problem (float64) with non-trivial norm gains."""
    A = len(lengths)
    cu = np.zeros(A + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    g = (lambda: rs.uniform(0.5, 1.5, size=d)) if gains_random else (lambda: np.ones(d))
    p = dict(
        A=A, m=m, H=H, d=d, n_heads=n_heads, gamma=gamma, ff=ff, cu=cu, eps=1e-6,
        taps=[rs.standard_normal((T, H)) for _ in range(m)],
        w_c=rs.standard_normal((m * H, d)) * w_std,
        ctx_norm=g(),
        block_in=rs.standard_normal((A, gamma, d)),
        block_pos=rs.standard_normal((gamma, d)) * 0.3,
        out_norm=g(),
        layers=[dict(attn_norm=g(), wq=rs.standard_normal((d, d)) * w_std,
                     wk=rs.standard_normal((d, d)) * w_std,
                     wv=rs.standard_normal((d, d)) * w_std,
                     wo=rs.standard_normal((d, d)) * w_std, ff_norm=g(),
                     w_gate=rs.standard_normal((d, ff)) * w_std,
                     w_up=rs.standard_normal((d, ff)) * w_std,
                     w_down=rs.standard_normal((ff, d)) * w_std)
                for _ in range(n_layers)],
    )
    return p


def _fwd(O, p, **kw):
    return O.block_forward(p["taps"], p["w_c"], p["ctx_norm"], p["cu"], p["block_in"],
                           p["block_pos"], p["layers"], p["out_norm"], p["n_heads"],
                           p["eps"], **kw)


# ---------------------------------------------------------------------------
# 1. brute force: every step as scalar Python loops
# ---------------------------------------------------------------------------

def _bf_matmul(X, W):
    n, k = len(X), len(W)
    mcols = len(W[0])
    return [[sum(X[i][t] * W[t][j] for t in range(k)) for j in range(mcols)] for i in range(n)]


def _bf_rms(row, g, eps):
    ms = sum(v * v for v in row) / len(row)
    s = 1.0 / math.sqrt(ms + eps)
    return [row[k] * s * g[k] for k in range(len(row))]


def brute_force_forward(p):
    """Scalar-loop forward of Eq 2, block init, Eq 3 + SiLU FFN, output norm."""
    A, gamma, d, n = p["A"], p["gamma"], p["d"], p["n_heads"]
    hd = d // n
    eps = p["eps"]
    cu = [int(c) for c in p["cu"]]
    T = cu[-1]
    taps = [t.tolist() for t in p["taps"]]
    X = [sum((taps[j][t] for j in range(p["m"])), []) for t in range(T)]
    P = _bf_matmul(X, p["w_c"].tolist())
    C = [_bf_rms(P[t], p["ctx_norm"].tolist(), eps) for t in range(T)]
    D = [[[p["block_in"][b, j, k] + p["block_pos"][j, k] for k in range(d)]
          for j in range(gamma)] for b in range(A)]
    for lw in p["layers"]:
        L = {k: v.tolist() for k, v in lw.items()}
        newD = []
        for b in range(A):
            U = [_bf_rms(D[b][j], L["attn_norm"], eps) for j in range(gamma)]
            ctx = C[cu[b]:cu[b + 1]]
            Uc = [_bf_rms(r, L["attn_norm"], eps) for r in ctx]
            Q = _bf_matmul(U, L["wq"])
            Kd, Vd = _bf_matmul(U, L["wk"]), _bf_matmul(U, L["wv"])
            Kc = _bf_matmul(Uc, L["wk"]) if Uc else []
            Vc = _bf_matmul(Uc, L["wv"]) if Uc else []
            keys, vals = Kc + Kd, Vc + Vd
            att = [[0.0] * d for _ in range(gamma)]
            for h in range(n):
                lo = h * hd
                for j in range(gamma):
                    s = [sum(Q[j][lo + c] * kk[lo + c] for c in range(hd)) / math.sqrt(hd)
                         for kk in keys]
                    mx = max(s)
                    e = [math.exp(v - mx) for v in s]
                    z = sum(e)
                    for c in range(hd):
                        att[j][lo + c] = sum(e[t] * vals[t][lo + c] for t in range(len(e))) / z
            ao = _bf_matmul(att, L["wo"])
            E = [[D[b][j][k] + ao[j][k] for k in range(d)] for j in range(gamma)]
            Z = [_bf_rms(E[j], L["ff_norm"], eps) for j in range(gamma)]
            G, Up = _bf_matmul(Z, L["w_gate"]), _bf_matmul(Z, L["w_up"])
            Hh = [[G[j][f] / (1.0 + math.exp(-G[j][f])) * Up[j][f] for f in range(len(G[j]))]
                  for j in range(gamma)]
            dn = _bf_matmul(Hh, L["w_down"])
            newD.append([[E[j][k] + dn[j][k] for k in range(d)] for j in range(gamma)])
        D = newD
    out = [[_bf_rms(D[b][j], p["out_norm"].tolist(), eps) for j in range(gamma)] for b in range(A)]
    return np.array(C, dtype=np.float64).reshape(T, d), np.array(out, dtype=np.float64)


def pin_brute_force(O, seed=0):
    rs = np.random.default_rng(seed)
    for lengths in ([3, 1], [0, 2], [4]):
        p = _rand_problem(rs, lengths=lengths)
        tr = {}
        out = _fwd(O, p, trace=tr)
        C_bf, out_bf = brute_force_forward(p)
        assert rel_err(tr["C"], C_bf) < TIGHT, ("brute force Eq 2", lengths)
        assert rel_err(out, out_bf) < TIGHT, ("brute force forward", lengths)


# ---------------------------------------------------------------------------
# 2. library routines: torch CPU float64 (independent implementation)
# ---------------------------------------------------------------------------

def torch_forward(p):
    import torch
    import torch.nn.functional as F
    t = lambda a: torch.as_tensor(np.asarray(a), dtype=torch.float64)
    eps, n = p["eps"], p["n_heads"]
    A, gamma, d = p["A"], p["gamma"], p["d"]
    hd = d // n
    cu = [int(c) for c in p["cu"]]
    X = torch.cat([t(x) for x in p["taps"]], dim=1)
    C = F.rms_norm(X @ t(p["w_c"]), (d,), weight=t(p["ctx_norm"]), eps=eps)
    D = t(p["block_in"]) + t(p["block_pos"])[None]
    for lw in p["layers"]:
        W = {k: t(v) for k, v in lw.items()}
        U = F.rms_norm(D, (d,), weight=W["attn_norm"], eps=eps)
        Uc = F.rms_norm(C, (d,), weight=W["attn_norm"], eps=eps)
        rows = []
        for b in range(A):
            q = (U[b] @ W["wq"]).view(gamma, n, hd).transpose(0, 1)
            kv_in = torch.cat([Uc[cu[b]:cu[b + 1]], U[b]], dim=0)
            k = (kv_in @ W["wk"]).view(-1, n, hd).transpose(0, 1)
            v = (kv_in @ W["wv"]).view(-1, n, hd).transpose(0, 1)
            o = F.scaled_dot_product_attention(q, k, v, is_causal=False)
            rows.append(o.transpose(0, 1).reshape(gamma, d))
        E = D + torch.stack(rows) @ W["wo"]
        Z = F.rms_norm(E, (d,), weight=W["ff_norm"], eps=eps)
        D = E + (F.silu(Z @ W["w_gate"]) * (Z @ W["w_up"])) @ W["w_down"]
    out = F.rms_norm(D, (d,), weight=t(p["out_norm"]), eps=eps)
    return C.numpy(), out.numpy()


def pin_torch_library(O, seed=1):
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[7, 0, 12], m=3, H=8, d=32, n_heads=4, gamma=4,
                      n_layers=2, ff=64, w_std=0.3)
    tr = {}
    out = _fwd(O, p, trace=tr)
    C_t, out_t = torch_forward(p)
    assert rel_err(tr["C"], C_t) < TIGHT, "torch Eq 2"
    assert rel_err(out, out_t) < TIGHT, "torch forward"


# ---------------------------------------------------------------------------
# 3. closed forms
# ---------------------------------------------------------------------------

def pin_wq_zero_is_mean_of_values(O, seed=2):
    """W_Q = 0 makes every score 0, so each head returns the mean of its
    L_b + gamma value rows."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[5, 0, 3], d=8, n_heads=2, n_layers=1)
    lw = dict(p["layers"][0])
    lw["wq"] = np.zeros_like(lw["wq"])
    C = O.ctx_fuse(p["taps"], p["w_c"], p["ctx_norm"], p["eps"])
    D = O.block_init(p["block_in"], p["block_pos"])
    inter = {}
    O.block_layer(C, p["cu"], D, lw, p["n_heads"], p["eps"], intermediates=inter)
    cu = p["cu"]
    for b in range(p["A"]):
        vals = np.concatenate([inter["Vc"][cu[b]:cu[b + 1]], inter["Vd"][b]], axis=0)
        mean = vals.mean(axis=0)
        for j in range(p["gamma"]):
            assert rel_err(inter["Attn"][b, j], mean) < TIGHT, "W_Q=0 mean of V"


def pin_two_key_logistic(O, seed=3):
    """One context key and one block key: the context weight is the logistic
    sigma(s_c - s_d) of the score difference."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[1], d=6, n_heads=1, gamma=1, n_layers=1)
    C = O.ctx_fuse(p["taps"], p["w_c"], p["ctx_norm"], p["eps"])
    D = O.block_init(p["block_in"], p["block_pos"])
    inter = {}
    O.block_layer(C, p["cu"], D, p["layers"][0], 1, p["eps"], intermediates=inter)
    q, kc, kd = inter["Q"][0, 0], inter["Kc"][0], inter["Kd"][0, 0]
    vc, vd = inter["Vc"][0], inter["Vd"][0, 0]
    sc, sd = q @ kc / math.sqrt(6), q @ kd / math.sqrt(6)
    w = 1.0 / (1.0 + math.exp(-(sc - sd)))
    assert rel_err(inter["Attn"][0, 0], w * vc + (1 - w) * vd) < TIGHT, "two-key logistic"


def pin_residual_passthrough(O, seed=4):
    """W_O = 0 and W_down = 0 leave the block rows unchanged through every
    layer, so out = RMSNorm(block_in + block_pos; out_norm)."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[4, 2], n_layers=3)
    for lw in p["layers"]:
        lw["wo"] = np.zeros_like(lw["wo"])
        lw["w_down"] = np.zeros_like(lw["w_down"])
    out = _fwd(O, p)
    D0 = p["block_in"] + p["block_pos"][None]
    ms = np.mean(D0 ** 2, axis=-1, keepdims=True)
    ref = D0 / np.sqrt(ms + p["eps"]) * p["out_norm"]
    assert rel_err(out, ref) < TIGHT, "residual passthrough"


def pin_hand_example(O):
    """A one-row, one-head case worked by hand (eps = 0, identity weights).

    taps [3] and [4] with W_c = I give P = [3, 4], mean square 12.5, so
    C = [3, 4] / sqrt(12.5) (unit gains), whose mean square is exactly 1.
    Block row [1, 1] normalises to itself. Scores: context (3+4)/sqrt(12.5)/sqrt(2)
    = 7/5; block 2/sqrt(2) = sqrt(2). The context weight is
    1 / (1 + exp(sqrt(2) - 1.4)).
    """
    eye = np.eye(2)
    lw = dict(attn_norm=np.ones(2), wq=eye, wk=eye, wv=eye, wo=eye, ff_norm=np.ones(2),
              w_gate=eye, w_up=eye, w_down=eye)
    taps = [np.array([[3.0]]), np.array([[4.0]])]
    tr = {}
    out = O.block_forward(taps, eye, np.ones(2), [0, 1], np.array([[[1.0, 1.0]]]),
                          np.zeros((1, 2)), [lw], np.ones(2), 1, 0.0, trace=tr)
    C = np.array([3.0, 4.0]) / math.sqrt(12.5)
    assert rel_err(tr["C"][0], C) < 1e-15
    pc = 1.0 / (1.0 + math.exp(math.sqrt(2.0) - 1.4))
    attn = pc * C + (1 - pc) * np.array([1.0, 1.0])
    E = np.array([1.0, 1.0]) + attn
    Z = E / math.sqrt(np.mean(E * E))
    D1 = E + Z / (1.0 + np.exp(-Z)) * Z
    ref = D1 / math.sqrt(np.mean(D1 * D1))
    assert rel_err(tr["D"][1][0, 0], D1) < 1e-14, "hand example, layer"
    assert rel_err(out[0, 0], ref) < 1e-14, "hand example, out"


# ---------------------------------------------------------------------------
# 4. invariants
# ---------------------------------------------------------------------------

def pin_scale_invariance(O, seed=5):
    """Eq 2 normalises each row: with eps = 0, scaling all m taps of a row by
    alpha leaves that row of H_ctx unchanged (the outlier rows)."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[6])
    C0 = O.ctx_fuse(p["taps"], p["w_c"], p["ctx_norm"], 0.0)
    taps = [t.copy() for t in p["taps"]]
    for t in taps:
        t[2] *= 8.0
        t[4] *= 0.125
    C1 = O.ctx_fuse(taps, p["w_c"], p["ctx_norm"], 0.0)
    assert rel_err(C1, C0) < 1e-14, "scale invariance"


def pin_block_permutation(O, seed=6):
    """Bidirectional block: permuting block rows of block_in and block_pos
    together permutes the outputs the same way."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[5, 3], gamma=4)
    out = _fwd(O, p)
    perm = np.array([2, 0, 3, 1])
    q = dict(p)
    q["block_in"] = p["block_in"][:, perm]
    q["block_pos"] = p["block_pos"][perm]
    out2 = _fwd(O, q)
    assert rel_err(out2, out[:, perm]) < TIGHT, "block permutation"


def pin_context_permutation(O, seed=7):
    """The context carries no position: permuting a sequence's context rows
    (all taps together) leaves the block outputs unchanged."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[5, 4])
    out = _fwd(O, p)
    perm = np.concatenate([rs.permutation(5), 5 + rs.permutation(4)])
    q = dict(p)
    q["taps"] = [t[perm] for t in p["taps"]]
    out2 = _fwd(O, q)
    assert rel_err(out2, out) < TIGHT, "context permutation"


def pin_varlen_equals_separate(O, seed=8):
    """A packed batch equals separate single-sequence runs."""
    rs = np.random.default_rng(seed)
    lengths = [3, 0, 6]
    p = _rand_problem(rs, lengths=lengths)
    out = _fwd(O, p)
    cu = p["cu"]
    for b in range(len(lengths)):
        q = dict(p)
        q["taps"] = [t[cu[b]:cu[b + 1]] for t in p["taps"]]
        q["cu"] = np.array([0, lengths[b]])
        q["block_in"] = p["block_in"][b:b + 1]
        q["A"] = 1
        ob = _fwd(O, q)
        assert rel_err(ob[0], out[b]) < TIGHT, ("varlen", b)


def _digest(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def pin_readonly_context(O, seed=9):
    """The context memory is read-only: block_layer never changes C, and every
    layer sees the same C."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[4, 2], n_layers=3)
    C = O.ctx_fuse(p["taps"], p["w_c"], p["ctx_norm"], p["eps"])
    h0 = _digest(C)
    D = O.block_init(p["block_in"], p["block_pos"])
    for lw in p["layers"]:
        D = O.block_layer(C, p["cu"], D, lw, p["n_heads"], p["eps"])
        assert _digest(C) == h0, "context modified"
    tr = {}
    out = _fwd(O, p, trace=tr)
    assert _digest(tr["C"]) == h0
    ref = O.rmsnorm(D, p["out_norm"], p["eps"])
    assert rel_err(out, ref) < TIGHT


def pin_empty_context_textbook(O, seed=10):
    """L_b = 0: the layer is a textbook pre-norm, non-causal transformer block
    with a SwiGLU FFN over the gamma block rows (torch.nn.MultiheadAttention
    with Q/K/V/O weights, no biases)."""
    import torch
    import torch.nn.functional as F
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[0, 0], d=8, n_heads=2, gamma=5, n_layers=2)
    out = _fwd(O, p)
    d = p["d"]
    t = lambda a: torch.as_tensor(np.asarray(a), dtype=torch.float64)
    D = t(p["block_in"]) + t(p["block_pos"])[None]
    for lw in p["layers"]:
        W = {k: t(v) for k, v in lw.items()}
        mha = torch.nn.MultiheadAttention(d, p["n_heads"], bias=False, batch_first=True,
                                          dtype=torch.float64)
        with torch.no_grad():
            mha.in_proj_weight.copy_(torch.cat([W["wq"].T, W["wk"].T, W["wv"].T], 0))
            mha.out_proj.weight.copy_(W["wo"].T)
        x = F.rms_norm(D, (d,), weight=W["attn_norm"], eps=p["eps"])
        with torch.no_grad():
            a, _ = mha(x, x, x, need_weights=False)
        E = D + a
        Z = F.rms_norm(E, (d,), weight=W["ff_norm"], eps=p["eps"])
        D = E + (F.silu(Z @ W["w_gate"]) * (Z @ W["w_up"])) @ W["w_down"]
    ref = F.rms_norm(D, (d,), weight=t(p["out_norm"]), eps=p["eps"]).numpy()
    assert rel_err(out, ref) < TIGHT, "empty context = textbook block"


def pin_fp32_close_to_fp64(O, seed=11):
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[40, 17], m=3, H=16, d=32, n_heads=4, gamma=5,
                      n_layers=3, ff=64, w_std=0.2)
    o64 = _fwd(O, p)
    o32 = _fwd(O, p, dtype=np.float32)
    assert o32.dtype == np.float32
    assert rel_err(o32, o64) < 1e-5, "fp32 mode"


def split_combine_attention(q, k, v, chunk):
    """Attention computed chunk by chunk with per-chunk (max, sum, output)
    partials merged by the log-sum-exp identity (the split-chunk attention
    plus combine of dspark-runtime.js). q [g, hd], k/v [n, hd]."""
    scale = 1.0 / math.sqrt(q.shape[1])
    parts = []
    for c0 in range(0, k.shape[0], chunk):
        s = (q @ k[c0:c0 + chunk].T) * scale
        mc = s.max(axis=1)
        e = np.exp(s - mc[:, None])
        parts.append((mc, e.sum(axis=1), e @ v[c0:c0 + chunk]))
    M = np.max([pt[0] for pt in parts], axis=0)
    l = sum(pt[1] * np.exp(pt[0] - M) for pt in parts)
    o = sum(pt[2] * np.exp(pt[0] - M)[:, None] for pt in parts)
    return o / l[:, None]


def pin_split_combine(O, seed=12):
    """The chunked (max, sum) merge equals the one-pass softmax attention for
    every chunk size from 1 to L + gamma."""
    rs = np.random.default_rng(seed)
    L, gamma, hd = 13, 3, 4
    Q = rs.standard_normal((1, gamma, hd)) * 2
    Kc, Vc = rs.standard_normal((L, hd)) * 2, rs.standard_normal((L, hd))
    Kd, Vd = rs.standard_normal((1, gamma, hd)) * 2, rs.standard_normal((1, gamma, hd))
    ref = O.attention(Q, Kc, Vc, Kd, Vd, [0, L], 1)[0]
    k = np.concatenate([Kc, Kd[0]])
    v = np.concatenate([Vc, Vd[0]])
    for chunk in range(1, L + gamma + 1):
        assert rel_err(split_combine_attention(Q[0], k, v, chunk), ref) < 1e-13, chunk


# ---------------------------------------------------------------------------
# 5. tanh-GELU (the gated FFN activation of module-dflash.ts, #layer)
# ---------------------------------------------------------------------------

def pin_gelu_tanh(O):
    """tanh-GELU against torch's independent implementation (float64,
    approximate="tanh"), and its closed forms: gelu(0) = 0, gelu(x) -> x for
    large x and -> 0 for large -x, gelu(x) - gelu(-x) = x (it is x * an odd
    sigmoid-like factor 0.5 (1 + tanh(.))), slope 1/2 at 0."""
    import torch
    import torch.nn.functional as F
    x = np.linspace(-8.0, 8.0, 2001)
    ref = F.gelu(torch.as_tensor(x, dtype=torch.float64), approximate="tanh").numpy()
    assert rel_err(O.gelu_tanh(x), ref) < 1e-14, "gelu vs torch"
    assert O.gelu_tanh(np.array([0.0]))[0] == 0.0
    big = np.array([30.0, 60.0])
    assert np.all(np.abs(O.gelu_tanh(big) - big) < 1e-12)
    assert np.all(np.abs(O.gelu_tanh(-big)) < 1e-12)
    assert np.max(np.abs(O.gelu_tanh(x) - O.gelu_tanh(-x) - x)) < 1e-12, "odd part"
    h = 1e-6
    slope = (O.gelu_tanh(np.array([h]))[0] - O.gelu_tanh(np.array([-h]))[0]) / (2 * h)
    assert abs(slope - 0.5) < 1e-9, slope


# ---------------------------------------------------------------------------
# 6. incremental context (dspark-runtime.js updateContext / store / propose)
# ---------------------------------------------------------------------------

def _append_in_pieces(O, p, pieces, dtype=np.float64):
    """Fill a cache through cache_append calls: ``pieces`` is a list of
    per-sequence row counts, consumed in order from each sequence's rows."""
    A, d = p["A"], p["d"]
    cache = O.DraftCache(A, len(p["layers"]), d, dtype=dtype)
    cu = [int(c) for c in p["cu"]]
    done = [0] * A
    for counts in pieces:
        rows = []
        cu_new = [0]
        for b in range(A):
            r0 = cu[b] + done[b]
            rows.append((r0, r0 + counts[b]))
            cu_new.append(cu_new[-1] + counts[b])
            done[b] += counts[b]
        taps_new = [np.concatenate([t[r0:r1] for r0, r1 in rows], axis=0) for t in p["taps"]]
        O.cache_append(cache, taps_new, cu_new, p["w_c"], p["ctx_norm"], p["layers"], p["eps"])
    assert done == [cu[b + 1] - cu[b] for b in range(A)]
    return cache


def pin_cache_equals_full_context(O, seed=20):
    """The context is read-only memory that every layer re-projects (the
    module-dflash.ts header): a cache filled by several appends of any sizes,
    empty ones included, gives the same draft block as the scalar-loop
    forward over the whole context."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[5, 0, 3])
    cache = _append_in_pieces(O, p, [[2, 0, 0], [0, 0, 3], [3, 0, 0], [0, 0, 0]])
    assert list(cache.lengths()) == [5, 0, 3]
    out = O.block_propose(cache, p["block_in"], p["block_pos"], p["layers"], p["out_norm"],
                          p["n_heads"], p["eps"])
    _, out_bf = brute_force_forward(p)
    assert rel_err(out, out_bf) < TIGHT, "incremental vs brute force"


def pin_cache_rows_are_row_local(O, seed=21):
    """Each cached row depends on its own context row only: appending rows
    one at a time fills the cache with the same keys and values as one
    append of all of them, and a sequence's rows are unaffected by the rows
    appended to the other sequences."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[4, 2], n_layers=2)
    whole = _append_in_pieces(O, p, [[4, 2]])
    single = _append_in_pieces(O, p, [[1, 0]] * 4 + [[0, 1]] * 2)
    for b in range(2):
        for i in range(2):
            assert rel_err(single.K[b][i], whole.K[b][i]) < TIGHT
            assert rel_err(single.V[b][i], whole.V[b][i]) < TIGHT
    alone = O.DraftCache(1, 2, p["d"])
    O.cache_append(alone, [t[:4] for t in p["taps"]], [0, 4], p["w_c"], p["ctx_norm"],
                   p["layers"], p["eps"])
    assert rel_err(alone.K[0][1], whole.K[0][1]) < TIGHT


# ---------------------------------------------------------------------------
# 7. Markov head, confidence head, greedy loop (module-dflash.ts forwardInfer)
# ---------------------------------------------------------------------------

def _markov_problem(rs, A=2, G=4, d=6, r=3, V=11):
    return dict(block=rs.standard_normal((A, G, d)), U=rs.standard_normal((A, G, V)),
                anchor=rs.integers(0, V, size=A), w1=rs.standard_normal((V, r)),
                w2=rs.standard_normal((r, V)), cw=rs.standard_normal(d + r) * 0.5, cb=0.3)


def _markov_brute(q):
    """Scalar loops over forwardInfer's per-position steps."""
    A, G, d = q["block"].shape
    V, r = q["w1"].shape
    toks, conf = [], []
    for b in range(A):
        prev = int(q["anchor"][b])
        tb, cb = [], []
        for k in range(G):
            e1 = [q["w1"][prev][i] for i in range(r)]
            lg = [q["U"][b][k][v] + sum(e1[i] * q["w2"][i][v] for i in range(r)) for v in range(V)]
            best = 0
            for v in range(1, V):
                if lg[v] > lg[best]:
                    best = v
            z = sum(q["block"][b][k][i] * q["cw"][i] for i in range(d))
            z += sum(e1[i] * q["cw"][d + i] for i in range(r)) + q["cb"]
            cb.append(1.0 / (1.0 + math.exp(-z)))
            tb.append(best)
            prev = best
        toks.append(tb)
        conf.append(cb)
    return np.array(toks), np.array(conf)


def _markov(O, q, **kw):
    return O.markov_draft(q["block"], q["U"], q["anchor"], q["w1"], q["w2"], q["cw"], q["cb"], **kw)


def pin_markov_brute_force(O, seed=30):
    rs = np.random.default_rng(seed)
    q = _markov_problem(rs)
    toks, conf, _ = _markov(O, q)
    bt, bc = _markov_brute(q)
    assert np.array_equal(toks, bt), (toks, bt)
    assert rel_err(conf, bc) < TIGHT


def pin_markov_closed_forms(O, seed=31):
    """W2 = 0 (the initialisation of initFromDims, "pure parallel DFlash")
    gives token k = argmax of the base logits at position k; conf.w = 0 and
    conf.b = 0 give confidence sigmoid(0) = 1/2 exactly; equal maxima resolve
    to the lowest index."""
    rs = np.random.default_rng(seed)
    q = _markov_problem(rs)
    q["w2"] = np.zeros_like(q["w2"])
    toks, _, logits = _markov(O, q)
    assert np.array_equal(toks, np.argmax(q["U"], axis=-1))
    assert np.array_equal(logits, q["U"])
    q["cw"] = np.zeros_like(q["cw"])
    q["cb"] = 0.0
    assert np.all(_markov(O, q)[1] == 0.5)
    U = np.zeros_like(q["U"])
    U[..., 7] = 2.0
    U[..., 3] = 2.0
    U[..., 9] = 1.0
    q["U"] = U
    assert np.all(_markov(O, q)[0] == 3), "ties go to the lowest index"


def pin_markov_chain_feeds_back(O, seed=32):
    """The previous token drives the next position: with zero base logits,
    one-hot Markov embeddings (w1 = identity, r = V) and w2 the cyclic shift
    v -> v + 1, the greedy draft counts up from the anchor token."""
    rs = np.random.default_rng(seed)
    V, A, G, d = 9, 3, 6, 4
    q = dict(block=rs.standard_normal((A, G, d)), U=np.zeros((A, G, V)),
             anchor=np.array([0, 4, 8]), w1=np.eye(V), w2=np.roll(np.eye(V), 1, axis=1),
             cw=np.zeros(d + V), cb=0.0)
    toks, _, _ = _markov(O, q)
    want = (q["anchor"][:, None] + np.arange(1, G + 1)[None, :]) % V
    assert np.array_equal(toks, want), (toks, want)


def pin_markov_confidence_torch(O, seed=33):
    """The confidence head against torch (float64 sigmoid of a linear map of
    [block row, Markov embedding of the previous token])."""
    import torch
    rs = np.random.default_rng(seed)
    q = _markov_problem(rs)
    toks, conf, _ = _markov(O, q)
    prev = np.concatenate([q["anchor"][:, None], toks[:, :-1]], axis=1)
    x = np.concatenate([q["block"], q["w1"][prev]], axis=-1)
    ref = torch.sigmoid(torch.as_tensor(x) @ torch.as_tensor(q["cw"]) + q["cb"]).numpy()
    assert rel_err(conf, ref) < TIGHT


# ---------------------------------------------------------------------------
# 8. block construction and the padded-batch mask (#buildBlock, #maskBias)
# ---------------------------------------------------------------------------

def pin_build_block_brute_force(O, seed=40):
    rs = np.random.default_rng(seed)
    A, H, d, G = 3, 5, 4, 4
    ae, tp = rs.standard_normal((A, H)), rs.standard_normal((H, d))
    me, bp = rs.standard_normal((G - 1, d)), rs.standard_normal((G, d))
    Hd = O.build_block(ae, tp, me, bp)
    for b in range(A):
        for k in range(d):
            v = sum(ae[b][i] * tp[i][k] for i in range(H)) + bp[0][k]
            assert abs(Hd[b, 0, k] - v) < 1e-12
            for j in range(1, G):
                assert abs(Hd[b, j, k] - (me[j - 1][k] + bp[j][k])) < 1e-15
    one = O.build_block(ae, tp, me[:0], bp[:1])
    assert one.shape == (A, 1, d)


def _padded_from_packed(p, rs, Lctx, real_rows_first=False):
    """A padded batch [A, Lctx, H] holding each sequence's real rows at
    random (or leading) positions, padding rows filled with noise."""
    A, m = p["A"], p["m"]
    cu = [int(c) for c in p["cu"]]
    mask = np.zeros((A, Lctx))
    taps = [rs.standard_normal((A, Lctx, p["H"])) * 3.0 for _ in range(m)]
    for b in range(A):
        L = cu[b + 1] - cu[b]
        pos = np.arange(L) if real_rows_first else np.sort(rs.choice(Lctx, size=L, replace=False))
        mask[b, pos] = 1
        for j in range(m):
            taps[j][b, pos] = p["taps"][j][cu[b]:cu[b + 1]]
    return taps, mask


def pin_padded_mask_equals_packed(O, seed=41):
    """#maskBias: padding rows get a -1e9 bias, so a padded batch gives the
    packed (varlen) result of its real rows, wherever the padding sits (the
    context carries no position); an all-ones mask adds nothing."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[3, 0, 5])
    ref = _fwd(O, p)
    for lead in (True, False):
        taps, mask = _padded_from_packed(p, rs, 7, real_rows_first=lead)
        out = O.block_forward_padded(taps, p["w_c"], p["ctx_norm"], mask, p["block_in"],
                                     p["block_pos"], p["layers"], p["out_norm"], p["n_heads"],
                                     p["eps"])
        assert rel_err(out, ref) < TIGHT, lead
    assert np.all(O.mask_bias(np.ones((2, 5)), 3) == 0.0)
    b = O.mask_bias(np.array([[1, 0, 1]]), 2)
    assert b.tolist() == [[0.0, -1e9, 0.0, 0.0, 0.0]]


def pin_padded_bias_is_exact_in_float32(O, seed=42):
    """In float32 the -1e9 bias makes a padding key's weight exactly 0
    (exp underflows), so the float32 padded forward equals the float32
    packed forward up to float32 rounding."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[4, 6])
    taps, mask = _padded_from_packed(p, rs, 9)
    out = O.block_forward_padded(taps, p["w_c"], p["ctx_norm"], mask, p["block_in"],
                                 p["block_pos"], p["layers"], p["out_norm"], p["n_heads"],
                                 p["eps"], dtype=np.float32)
    assert rel_err(out, _fwd(O, p)) < 1e-5
    assert np.exp(np.float32(-1e9) + np.float32(50.0) - np.float32(60.0)) == 0.0


# ---------------------------------------------------------------------------
# 9. the page-1 layer variant (q/k norms, RoPE, grouped K/V heads, plain
#    context K/V)
# ---------------------------------------------------------------------------

def _variant_problem(rs, lengths, n_heads=4, n_kv=2, hd=4, n_layers=2, m=2, H=3, gamma=3, ff=6):
    d = n_heads * hd
    kvd = n_kv * hd
    p = _rand_problem(rs, lengths=lengths, m=m, H=H, d=d, n_heads=n_heads, gamma=gamma,
                      n_layers=n_layers, ff=ff)
    for lw in p["layers"]:
        lw["wk"] = rs.standard_normal((d, kvd)) * 0.5
        lw["wv"] = rs.standard_normal((d, kvd)) * 0.5
        lw["q_norm"] = rs.uniform(0.5, 1.5, size=hd)
        lw["k_norm"] = rs.uniform(0.5, 1.5, size=hd)
    p["n_kv"] = n_kv
    return p


def _vfwd(O, p, **kw):
    return O.variant_forward(p["taps"], p["w_c"], p["ctx_norm"], p["cu"], p["block_in"],
                             p["block_pos"], p["layers"], p["out_norm"], p["n_heads"],
                             p["n_kv"], p["eps"], **kw)


def pin_variant_reduces_to_layer(O, seed=50):
    """With every variant switch off (context norm on, no q/k norms, no RoPE,
    as many K/V heads as query heads) the variant is #layer itself."""
    rs = np.random.default_rng(seed)
    p = _rand_problem(rs, lengths=[4, 0, 2])
    p["n_kv"] = p["n_heads"]
    assert rel_err(_vfwd(O, p), _fwd(O, p)) < TIGHT


def pin_rope_closed_forms(O, seed=51):
    """RoPE as complex multiplication: the pair (x_c, x_{c+hd/2}) is the
    complex number x_c + i x_{c+hd/2} times exp(i pos theta^(-2c/hd)). So it is
    the identity at position 0, keeps norms, and q.k after rotation depends
    only on the difference of the two positions."""
    rs = np.random.default_rng(seed)
    hd, n, theta = 8, 5, 10000.0
    x = rs.standard_normal((n, hd))
    pos = rs.integers(0, 5000, size=n)
    z = x[:, :hd // 2] + 1j * x[:, hd // 2:]
    w = np.exp(1j * pos[:, None] * theta ** (-2.0 * np.arange(hd // 2) / hd)[None, :])
    zr = z * w
    ref = np.concatenate([zr.real, zr.imag], axis=1)
    assert rel_err(O.rope(x, pos, theta), ref) < 1e-12
    assert rel_err(O.rope(x, np.zeros(n, dtype=np.int64), theta), x) == 0.0
    assert rel_err(np.linalg.norm(O.rope(x, pos, theta), axis=1), np.linalg.norm(x, axis=1)) < 1e-13
    q, k = rs.standard_normal((1, hd)), rs.standard_normal((1, hd))
    for shift in (0, 7, 1234):
        a = O.rope(q, np.array([10 + shift]), theta) @ O.rope(k, np.array([3 + shift]), theta).T
        if shift == 0:
            a0 = a
        assert abs(a - a0).max() < 1e-10


def pin_variant_rope_shift_invariance(O, seed=52):
    """Positions count from each sequence's own start (context row t at t,
    block row j at L_b + j), and RoPE depends on position differences only:
    two sequences with equal contexts and blocks get equal drafts wherever
    they sit in the packed batch. Unlike the base method, the context then
    carries position: reordering a sequence's context rows changes its
    draft."""
    rs = np.random.default_rng(seed)
    p = _variant_problem(rs, lengths=[3, 3])
    for j in range(p["m"]):
        p["taps"][j][3:6] = p["taps"][j][0:3]
    p["block_in"][1] = p["block_in"][0]
    out = _vfwd(O, p, qk_norm=True, theta=100.0, ctx_norm_kv=False)
    assert rel_err(out[1], out[0]) < TIGHT
    # and RoPE does matter: a context row moved within its sequence changes the draft
    q = _variant_problem(np.random.default_rng(seed), lengths=[3, 3])
    for j in range(q["m"]):
        q["taps"][j][3:6] = q["taps"][j][[1, 0, 2]]
    q["block_in"][1] = q["block_in"][0]
    out2 = _vfwd(O, q, qk_norm=True, theta=100.0, ctx_norm_kv=False)
    assert rel_err(out2[1], out2[0]) > 1e-6


def pin_variant_gqa_is_repeated_heads(O, seed=53):
    """Grouped K/V heads (query head h reads K/V head h // (n / n_kv)) equal
    the full-head layer whose W_K / W_V repeat each K/V head's columns for
    the query heads of its group; likewise with q/k norms and RoPE."""
    rs = np.random.default_rng(seed)
    p = _variant_problem(rs, lengths=[4, 1], n_heads=4, n_kv=2, hd=4)
    full = {k: (v if not isinstance(v, list) else v) for k, v in p.items()}
    grp = p["n_heads"] // p["n_kv"]
    hd = p["d"] // p["n_heads"]
    full["layers"] = []
    for lw in p["layers"]:
        f = dict(lw)
        cols = np.concatenate([np.arange((h // grp) * hd, (h // grp + 1) * hd) for h in range(p["n_heads"])])
        f["wk"], f["wv"] = lw["wk"][:, cols], lw["wv"][:, cols]
        full["layers"].append(f)
    full["n_kv"] = p["n_heads"]
    for kw in (dict(), dict(qk_norm=True, theta=500.0)):
        assert rel_err(_vfwd(O, p, **kw), _vfwd(O, full, **kw)) < TIGHT, kw


def pin_variant_head_norm_torch(O, seed=54):
    """q_norm / k_norm are RMSNorms over each head (torch rms_norm over the
    last axis of the [.., heads, hd] view); with them, scaling W_Q and W_K
    by any positive factor leaves the draft unchanged (eps = 0)."""
    import torch
    import torch.nn.functional as F
    rs = np.random.default_rng(seed)
    x, g = rs.standard_normal((5, 12)), rs.uniform(0.5, 1.5, size=4)
    ref = F.rms_norm(torch.as_tensor(x).view(5, 3, 4), (4,), weight=torch.as_tensor(g), eps=1e-6)
    assert rel_err(O.head_rmsnorm(x, g, 3, 1e-6), ref.reshape(5, 12).numpy()) < 1e-14
    p = _variant_problem(rs, lengths=[3, 2])
    p["eps"] = 0.0
    out = _vfwd(O, p, qk_norm=True, theta=50.0)
    for lw in p["layers"]:
        lw["wq"] = lw["wq"] * 3.7
        lw["wk"] = lw["wk"] * 0.21
    assert rel_err(_vfwd(O, p, qk_norm=True, theta=50.0), out) < 1e-10


def pin_variant_plain_context_kv(O, seed=55):
    """Without the per-layer context norm the context rows enter W_K / W_V as
    Eq 2 leaves them. Eq 2's rows have RMS 1 (eps = 0, gain 1), so with unit
    attention-norm gains the two readings agree; with other gains they do
    not."""
    rs = np.random.default_rng(seed)
    p = _variant_problem(rs, lengths=[3, 4])
    p["eps"] = 0.0
    p["ctx_norm"] = np.ones(p["d"])
    for lw in p["layers"]:
        lw["attn_norm"] = np.ones(p["d"])
    a = _vfwd(O, p, ctx_norm_kv=True, qk_norm=True, theta=30.0)
    b = _vfwd(O, p, ctx_norm_kv=False, qk_norm=True, theta=30.0)
    assert rel_err(a, b) < 1e-12
    for lw in p["layers"]:
        lw["attn_norm"] = rs.uniform(0.5, 1.5, size=p["d"])
    a = _vfwd(O, p, ctx_norm_kv=True)
    b = _vfwd(O, p, ctx_norm_kv=False)
    assert rel_err(a, b) > 1e-6


def _variant_brute(p, *, qk_norm, theta, ctx_norm_kv):
    """Scalar loops over the variant forward, with RoPE as a rotation of the
    complex number x_c + i x_{c+hd/2} by the angle pos * theta^(-2c/hd) at
    explicit positions (context row t of a sequence at t, block row j at
    L_b + j)."""
    A, G, d, n, nkv = p["A"], p["gamma"], p["d"], p["n_heads"], p["n_kv"]
    hd, grp, eps = d // n, n // nkv, p["eps"]
    cu = [int(c) for c in p["cu"]]
    C, _ = brute_force_forward(dict(p, layers=[]))
    C = C.tolist()
    D = [[[p["block_in"][b, j, k] + p["block_pos"][j, k] for k in range(d)] for j in range(G)]
         for b in range(A)]

    def head_norm(row, g, heads):
        out = []
        for h in range(heads):
            out += _bf_rms(row[h * hd:(h + 1) * hd], list(g), eps)
        return out

    def rot(row, pos, heads):
        out = list(row)
        for h in range(heads):
            for c in range(hd // 2):
                z = complex(row[h * hd + c], row[h * hd + c + hd // 2])
                ang = pos * theta ** (-2.0 * c / hd)
                z *= complex(math.cos(ang), math.sin(ang))
                out[h * hd + c], out[h * hd + c + hd // 2] = z.real, z.imag
        return out

    for lw in p["layers"]:
        L_ = {k: np.asarray(v).tolist() for k, v in lw.items()}
        newD = []
        for b in range(A):
            ctx = C[cu[b]:cu[b + 1]]
            xc = [_bf_rms(r, L_["attn_norm"], eps) for r in ctx] if ctx_norm_kv else ctx
            Kc = _bf_matmul(xc, L_["wk"]) if xc else []
            Vc = _bf_matmul(xc, L_["wv"]) if xc else []
            U = [_bf_rms(D[b][j], L_["attn_norm"], eps) for j in range(G)]
            Q, Kd, Vd = _bf_matmul(U, L_["wq"]), _bf_matmul(U, L_["wk"]), _bf_matmul(U, L_["wv"])
            if qk_norm:
                Kc = [head_norm(r, L_["k_norm"], nkv) for r in Kc]
                Q = [head_norm(r, L_["q_norm"], n) for r in Q]
                Kd = [head_norm(r, L_["k_norm"], nkv) for r in Kd]
            Lb = len(ctx)
            if theta > 0:
                Kc = [rot(r, t, nkv) for t, r in enumerate(Kc)]
                Q = [rot(r, Lb + j, n) for j, r in enumerate(Q)]
                Kd = [rot(r, Lb + j, nkv) for j, r in enumerate(Kd)]
            keys, vals = Kc + Kd, Vc + Vd
            att = [[0.0] * d for _ in range(G)]
            for h in range(n):
                qo, ko = h * hd, (h // grp) * hd
                for j in range(G):
                    sc = [sum(Q[j][qo + c] * kk[ko + c] for c in range(hd)) / math.sqrt(hd) for kk in keys]
                    mx = max(sc)
                    e = [math.exp(v - mx) for v in sc]
                    z = sum(e)
                    for c in range(hd):
                        att[j][qo + c] = sum(e[t] * vals[t][ko + c] for t in range(len(e))) / z
            ao = _bf_matmul(att, L_["wo"])
            E = [[D[b][j][k] + ao[j][k] for k in range(d)] for j in range(G)]
            Z = [_bf_rms(E[j], L_["ff_norm"], eps) for j in range(G)]
            Gt, Up = _bf_matmul(Z, L_["w_gate"]), _bf_matmul(Z, L_["w_up"])
            Hh = [[Gt[j][f] / (1.0 + math.exp(-Gt[j][f])) * Up[j][f] for f in range(len(Gt[j]))]
                  for j in range(G)]
            dn = _bf_matmul(Hh, L_["w_down"])
            newD.append([[E[j][k] + dn[j][k] for k in range(d)] for j in range(G)])
        D = newD
    return np.array([[_bf_rms(D[b][j], p["out_norm"].tolist(), eps) for j in range(G)] for b in range(A)])


def pin_variant_brute_force(O, seed=56):
    rs = np.random.default_rng(seed)
    p = _variant_problem(rs, lengths=[3, 0, 2], n_heads=4, n_kv=2, hd=4)
    for kw in (dict(qk_norm=True, theta=1000.0, ctx_norm_kv=False),
               dict(qk_norm=False, theta=77.0, ctx_norm_kv=True),
               dict(qk_norm=True, theta=0.0, ctx_norm_kv=True)):
        assert rel_err(_vfwd(O, p, **kw), _variant_brute(p, **kw)) < TIGHT, kw


ALL_PINS = [
    pin_brute_force, pin_torch_library, pin_wq_zero_is_mean_of_values,
    pin_two_key_logistic, pin_residual_passthrough, pin_hand_example,
    pin_scale_invariance, pin_block_permutation, pin_context_permutation,
    pin_varlen_equals_separate, pin_readonly_context, pin_empty_context_textbook,
    pin_fp32_close_to_fp64, pin_split_combine, pin_gelu_tanh,
    pin_cache_equals_full_context, pin_cache_rows_are_row_local,
    pin_markov_brute_force, pin_markov_closed_forms, pin_markov_chain_feeds_back,
    pin_markov_confidence_torch, pin_build_block_brute_force, pin_padded_mask_equals_packed,
    pin_padded_bias_is_exact_in_float32, pin_variant_reduces_to_layer, pin_rope_closed_forms,
    pin_variant_rope_shift_invariance, pin_variant_gqa_is_repeated_heads,
    pin_variant_head_norm_torch, pin_variant_plain_context_kv, pin_variant_brute_force,
]
