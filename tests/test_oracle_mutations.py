"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each of them. This shows the pins constrain every step of the
oracle: norms, projections, attention wiring, residuals, FFN and packing."""
import math

import numpy as np
import pytest

import oracle as O
import oracle.dspark_oracle as OM
import oracle_pins as P


def _attn_factory(*, scale_pow=-0.5, causal=False, cross_seq=False, swap_heads=False):
    def attention(Q, Kc, Vc, Kd, Vd, cu, n_heads):
        A, gamma, d = Q.shape
        hd = d // n_heads
        out = np.empty_like(Q)
        for b in range(A):
            r0, r1 = (0, int(cu[-1])) if cross_seq else (int(cu[b]), int(cu[b + 1]))
            for h in range(n_heads):
                cs = slice(h * hd, (h + 1) * hd)
                ks = slice((n_heads - 1 - h) * hd, (n_heads - h) * hd) if swap_heads else cs
                q = Q[b, :, cs]
                k = np.concatenate([Kc[r0:r1, ks], Kd[b, :, ks]], axis=0)
                v = np.concatenate([Vc[r0:r1, cs], Vd[b, :, cs]], axis=0)
                s = (q @ k.T) * hd ** scale_pow
                if causal:
                    L = r1 - r0
                    for j in range(gamma):
                        s[j, L + j + 1:] = -np.inf
                out[b, :, cs] = OM.softmax(s) @ v
        return out
    return attention


def _rms_no_gain(x, g, eps):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def _rms_eps_outside(x, g, eps):
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * g


def _rms_centered(x, g, eps):
    xc = x - x.mean(axis=-1, keepdims=True)
    return xc / np.sqrt(np.mean(xc * xc, axis=-1, keepdims=True) + eps) * g


def _rms_sum_not_mean(x, g, eps):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * g


def _layer_mutant(kind):
    orig = OM.block_layer

    def block_layer(C, cu, D, lw, n_heads, eps, dtype=np.float64, act="silu", intermediates=None):
        lw = dict(lw)
        if kind == "swap_kv":
            lw["wk"], lw["wv"] = lw["wv"], lw["wk"]
        elif kind == "transpose_wo":
            lw["wo"] = np.asarray(lw["wo"]).T
        elif kind == "swap_gate_up":
            lw["w_gate"], lw["w_up"] = lw["w_up"], lw["w_gate"]
        elif kind == "gelu":
            act = "gelu_tanh"
        elif kind == "ff_norm_is_attn_norm":
            lw["ff_norm"] = lw["attn_norm"]
        out = orig(C, cu, D, lw, n_heads, eps, dtype=dtype, act=act, intermediates=intermediates)
        if kind == "no_ffn_residual":
            inter = {}
            orig(C, cu, D, lw, n_heads, eps, dtype=dtype, act=act, intermediates=inter)
            out = out - inter["E"]
        return out
    return block_layer


def _layer_no_ctx_norm(C, cu, D, lw, n_heads, eps, dtype=np.float64, act="silu", intermediates=None):
    # the context rows enter W_K/W_V without the attention norm
    f = lambda a: np.asarray(a, dtype=dtype)
    D = f(D)
    U = OM.rmsnorm(D, f(lw["attn_norm"]), eps)
    Q, Kd, Vd = U @ f(lw["wq"]), U @ f(lw["wk"]), U @ f(lw["wv"])
    Kc, Vc = f(C) @ f(lw["wk"]), f(C) @ f(lw["wv"])
    Attn = OM.attention(Q, Kc, Vc, Kd, Vd, cu, n_heads)
    E = D + Attn @ f(lw["wo"])
    Z = OM.rmsnorm(E, f(lw["ff_norm"]), eps)
    out = E + (OM.silu(Z @ f(lw["w_gate"])) * (Z @ f(lw["w_up"]))) @ f(lw["w_down"])
    if intermediates is not None:
        intermediates.update(dict(Q=Q, Kd=Kd, Vd=Vd, Kc=Kc, Vc=Vc, Attn=Attn, E=E))
    return out


def _block_init_no_pos(block_in, block_pos, dtype=np.float64):
    return np.asarray(block_in, dtype=dtype)


def _ctx_fuse_reversed_taps(taps, w_c, ctx_norm, eps, dtype=np.float64):
    return OM.rmsnorm(np.concatenate([np.asarray(t, dtype) for t in taps[::-1]], 1) @ np.asarray(w_c, dtype),
                      np.asarray(ctx_norm, dtype), eps)


def _silu_sigmoid_only(x):
    return 1.0 / (1.0 + np.exp(-x))


def _gelu_wrong_coefficient(x):
    c = x.dtype.type(math.sqrt(2.0 / math.pi))
    return x.dtype.type(0.5) * x * (x.dtype.type(1.0) + np.tanh(c * (x + x.dtype.type(0.05) * x ** 3)))


def _gelu_sigmoid_form(x):
    return x / (1.0 + np.exp(-1.702 * x))


def _markov_factory(kind):
    def markov_draft(block, base_logits, anchor_tok, w1, w2, conf_w, conf_b, dtype=np.float64):
        f = lambda a: np.asarray(a, dtype=dtype)
        block, U, w1, w2, cw = f(block), f(base_logits), f(w1), f(w2), f(conf_w).reshape(-1)
        A, G, _ = block.shape
        toks = np.zeros((A, G), dtype=np.int64)
        conf = np.zeros((A, G))
        logits = np.zeros(U.shape)
        for b in range(A):
            prev = int(anchor_tok[b])
            for k in range(G):
                e1 = w1[prev]
                lk = U[b, k] + e1 @ w2
                tok = int(np.argmax(lk)) if kind != "last_tie" else int(len(lk) - 1 - np.argmax(lk[::-1]))
                ce = w1[tok] if kind == "conf_new_token" else e1
                z = np.concatenate([block[b, k], ce]) @ cw + conf_b
                conf[b, k] = 1.0 / (1.0 + np.exp(-z))
                logits[b, k] = lk
                toks[b, k] = tok
                if kind != "no_feedback":
                    prev = tok
        return toks, conf, logits
    return markov_draft


def _cache_append_no_norm(cache, taps_new, cu_new, w_c, ctx_norm, layers, eps):
    C = OM.ctx_fuse(taps_new, w_c, ctx_norm, eps)
    for i, lw in enumerate(layers):
        Kc, Vc = C @ lw["wk"], C @ lw["wv"]
        for b in range(len(cache.K)):
            r0, r1 = int(cu_new[b]), int(cu_new[b + 1])
            cache.K[b][i] = np.concatenate([cache.K[b][i], Kc[r0:r1]], axis=0)
            cache.V[b][i] = np.concatenate([cache.V[b][i], Vc[r0:r1]], axis=0)
    return C


def _cache_append_overwrites(cache, taps_new, cu_new, w_c, ctx_norm, layers, eps):
    C = OM.ctx_fuse(taps_new, w_c, ctx_norm, eps)
    for i, lw in enumerate(layers):
        Uc = OM.rmsnorm(C, lw["attn_norm"], eps)
        Kc, Vc = Uc @ lw["wk"], Uc @ lw["wv"]
        for b in range(len(cache.K)):
            r0, r1 = int(cu_new[b]), int(cu_new[b + 1])
            if r1 > r0:
                cache.K[b][i] = Kc[r0:r1]
                cache.V[b][i] = Vc[r0:r1]
    return C


def _build_block_no_pos0(anchor_emb, tok_proj, mask_emb, block_pos, dtype=np.float64):
    Hd = _ORIG_BUILD(anchor_emb, tok_proj, mask_emb, block_pos, dtype)
    Hd[:, 0] -= np.asarray(block_pos)[0]
    return Hd


def _build_block_pos_shift(anchor_emb, tok_proj, mask_emb, block_pos, dtype=np.float64):
    bp = np.asarray(block_pos)
    return _ORIG_BUILD(anchor_emb, tok_proj, mask_emb, np.roll(bp, 1, axis=0), dtype)


def _mask_bias_ignored(ctx_mask, gamma, dtype=np.float64):
    m = np.asarray(ctx_mask)
    return np.zeros((m.shape[0], m.shape[1] + gamma))


def _mask_bias_block_masked(ctx_mask, gamma, dtype=np.float64):
    m = np.asarray(ctx_mask, dtype=dtype)
    return np.concatenate([(m - 1.0) * 1e9, np.full((m.shape[0], gamma), -1e9)], axis=1)


def _rope_adjacent_pairs(x, pos, theta):
    hd = x.shape[-1]
    inv = theta ** (-2.0 * np.arange(hd // 2) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x1 * c - x2 * s
    out[..., 1::2] = x2 * c + x1 * s
    return out


def _rope_wrong_freq(x, pos, theta):
    hd = x.shape[-1]
    half = hd // 2
    inv = theta ** (-1.0 * np.arange(half) / hd)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _head_norm_whole_row(x, g, n_heads, eps):
    hd = x.shape[-1] // n_heads
    return OM.rmsnorm(x, np.tile(np.asarray(g), n_heads), eps)


def _variant_layer_factory(kind):
    """A copy of the variant layer with one planted mistake: query head h
    reading K/V head h % n_kv ("gqa_modulo"), or the block rows rotated at
    positions 0 .. gamma-1 instead of after their context ("block_pos_zero")."""
    def variant_layer(Kc, Vc, cu, D, lw, n_heads, n_kv_heads, eps, *, qk_norm, theta,
                      act="silu", dtype=np.float64):
        f = lambda a: np.asarray(a, dtype=dtype)
        D = f(D)
        A, G, d = D.shape
        hd = d // n_heads
        grp = n_heads // n_kv_heads
        U = OM.rmsnorm(D, f(lw["attn_norm"]), eps)
        Q, Kd, Vd = U @ f(lw["wq"]), U @ f(lw["wk"]), U @ f(lw["wv"])
        if qk_norm:
            Q = OM.head_rmsnorm(Q, lw["q_norm"], n_heads, eps)
            Kd = OM.head_rmsnorm(Kd, lw["k_norm"], n_kv_heads, eps)
        Attn = np.empty_like(Q)
        for b in range(A):
            r0, r1 = int(cu[b]), int(cu[b + 1])
            L = 0 if kind == "block_pos_zero" else r1 - r0
            qb, kdb = Q[b], Kd[b]
            if theta > 0:
                bpos = np.arange(L, L + G, dtype=np.int64)
                qb = OM._positions_rows(qb, n_heads, bpos, theta)
                kdb = OM._positions_rows(kdb, n_kv_heads, bpos, theta)
            for h in range(n_heads):
                kh = h % n_kv_heads if kind == "gqa_modulo" else h // grp
                qs, ks = slice(h * hd, (h + 1) * hd), slice(kh * hd, (kh + 1) * hd)
                k = np.concatenate([f(Kc)[r0:r1, ks], kdb[:, ks]], axis=0)
                v = np.concatenate([f(Vc)[r0:r1, ks], Vd[b][:, ks]], axis=0)
                Attn[b, :, qs] = OM.softmax((qb[:, qs] @ k.T) / math.sqrt(hd)) @ v
        E = D + Attn @ f(lw["wo"])
        Z = OM.rmsnorm(E, f(lw["ff_norm"]), eps)
        g = Z @ f(lw["w_gate"])
        a = OM.silu(g) if act == "silu" else OM.gelu_tanh(g)
        return E + (a * (Z @ f(lw["w_up"]))) @ f(lw["w_down"])
    return variant_layer


def _variant_ctx_kv_ignores_flag(C, cu, lw, n_kv_heads, eps, *, ctx_norm_kv, qk_norm, theta,
                                 dtype=np.float64):
    return _ORIG_VCTX(C, cu, lw, n_kv_heads, eps, ctx_norm_kv=True, qk_norm=qk_norm, theta=theta,
                      dtype=dtype)


def _variant_ctx_kv_no_knorm(C, cu, lw, n_kv_heads, eps, *, ctx_norm_kv, qk_norm, theta,
                             dtype=np.float64):
    return _ORIG_VCTX(C, cu, lw, n_kv_heads, eps, ctx_norm_kv=ctx_norm_kv, qk_norm=False,
                      theta=theta, dtype=dtype)


def _variant_ctx_kv_global_pos(C, cu, lw, n_kv_heads, eps, *, ctx_norm_kv, qk_norm, theta,
                               dtype=np.float64):
    # positions over the packed axis instead of each sequence's own
    return _ORIG_VCTX(C, [0, int(cu[-1])], lw, n_kv_heads, eps, ctx_norm_kv=ctx_norm_kv,
                      qk_norm=qk_norm, theta=theta, dtype=dtype)


_ORIG_BUILD = OM.build_block
_ORIG_VLAYER = OM.variant_layer
_ORIG_VCTX = OM.variant_context_kv


MUTANTS = {
    "no_softmax_scale": [("attention", _attn_factory(scale_pow=0.0))],
    "scale_1_over_hd": [("attention", _attn_factory(scale_pow=-1.0))],
    "causal_block": [("attention", _attn_factory(causal=True))],
    "cross_sequence_context": [("attention", _attn_factory(cross_seq=True))],
    "head_index_mixup": [("attention", _attn_factory(swap_heads=True))],
    "rms_ignores_gain": [("rmsnorm", _rms_no_gain)],
    "rms_eps_outside_sqrt": [("rmsnorm", _rms_eps_outside)],
    "rms_mean_centred": [("rmsnorm", _rms_centered)],
    "rms_sum_not_mean": [("rmsnorm", _rms_sum_not_mean)],
    "swap_wk_wv": [("block_layer", _layer_mutant("swap_kv"))],
    "transposed_wo": [("block_layer", _layer_mutant("transpose_wo"))],
    "swap_gate_up": [("block_layer", _layer_mutant("swap_gate_up"))],
    "gelu_not_silu": [("block_layer", _layer_mutant("gelu"))],
    "wrong_ff_norm": [("block_layer", _layer_mutant("ff_norm_is_attn_norm"))],
    "dropped_ffn_residual": [("block_layer", _layer_mutant("no_ffn_residual"))],
    "context_not_normalised": [("block_layer", _layer_no_ctx_norm)],
    "block_pos_dropped": [("block_init", _block_init_no_pos)],
    "taps_reversed": [("ctx_fuse", _ctx_fuse_reversed_taps)],
    "silu_missing_x": [("silu", _silu_sigmoid_only)],
    "gelu_wrong_coefficient": [("gelu_tanh", _gelu_wrong_coefficient)],
    "gelu_sigmoid_form": [("gelu_tanh", _gelu_sigmoid_form)],
    "markov_no_feedback": [("markov_draft", _markov_factory("no_feedback"))],
    "markov_conf_new_token": [("markov_draft", _markov_factory("conf_new_token"))],
    "markov_last_index_on_ties": [("markov_draft", _markov_factory("last_tie"))],
    "cache_context_not_normalised": [("cache_append", _cache_append_no_norm)],
    "cache_overwrites_instead_of_append": [("cache_append", _cache_append_overwrites)],
    "build_block_no_pos_on_anchor": [("build_block", _build_block_no_pos0)],
    "build_block_positions_shifted": [("build_block", _build_block_pos_shift)],
    "mask_bias_ignored": [("mask_bias", _mask_bias_ignored)],
    "mask_bias_masks_block": [("mask_bias", _mask_bias_block_masked)],
    "rope_adjacent_pairs": [("rope", _rope_adjacent_pairs)],
    "rope_wrong_frequencies": [("rope", _rope_wrong_freq)],
    "head_norm_over_whole_row": [("head_rmsnorm", _head_norm_whole_row)],
    "gqa_head_modulo": [("variant_layer", _variant_layer_factory("gqa_modulo"))],
    "block_rope_from_zero": [("variant_layer", _variant_layer_factory("block_pos_zero"))],
    "variant_ignores_context_norm_flag": [("variant_context_kv", _variant_ctx_kv_ignores_flag)],
    "variant_context_without_k_norm": [("variant_context_kv", _variant_ctx_kv_no_knorm)],
    "variant_context_global_positions": [("variant_context_kv", _variant_ctx_kv_global_pos)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    for attr, fn in MUTANTS[name]:
        monkeypatch.setattr(OM, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(OM)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
