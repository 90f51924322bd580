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


ALL_PINS = [
    pin_brute_force, pin_torch_library, pin_wq_zero_is_mean_of_values,
    pin_two_key_logistic, pin_residual_passthrough, pin_hand_example,
    pin_scale_invariance, pin_block_permutation, pin_context_permutation,
    pin_varlen_equals_separate, pin_readonly_context, pin_empty_context_textbook,
    pin_fp32_close_to_fp64, pin_split_combine,
]
