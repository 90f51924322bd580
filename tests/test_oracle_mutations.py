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
