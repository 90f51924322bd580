"""The layer variant of the page "src/dspark-runtime.js" (q/k norms, rotary
positions, grouped K/V heads, context K/V without the per-layer norm,
tanh-GELU FFN) against the oracle's variant_forward, through the C ABI: the
whole forward, one layer, and propose over a draft cache."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import TOL, Uploaded, rel_err

torch = pytest.importorskip("torch")
B = pytest.importorskip("block_draft_context_amd")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"

CASES = {
    # name: (workload kwargs, lengths, n_kv, switches)
    "bf16-all": (dict(name="v1", seed_id=101, A=3, m=2, H=128, d=512, n_heads=4, gamma=5, n_layers=2,
                      ff=1024, dtype="bf16"), [700, 0, 1200], 2,
                 dict(qk_norm=True, plain_ctx_kv=True, gelu_ffn=True, rope_theta=10000.0)),
    "bf16-rope-gqa4": (dict(name="v2", seed_id=102, A=2, m=2, H=128, d=1024, n_heads=8, gamma=4, n_layers=1,
                            ff=1024, dtype="bf16"), [3000, 517], 2, dict(rope_theta=1e6)),
    "bf16-qknorm-only": (dict(name="v3", seed_id=103, A=2, m=1, H=64, d=256, n_heads=2, gamma=6, n_layers=2,
                              ff=512, dtype="bf16"), [900, 64], 2, dict(qk_norm=True)),
    "bf16-gelu-plain": (dict(name="v4", seed_id=104, A=1, m=2, H=128, d=256, n_heads=2, gamma=5, n_layers=2,
                             ff=512, dtype="bf16"), [2000], 2, dict(gelu_ffn=True, plain_ctx_kv=True)),
    "f32-all-hd32": (dict(name="v5", seed_id=105, A=2, m=1, H=64, d=256, n_heads=8, gamma=3, n_layers=1,
                          ff=256, dtype="f32"), [300, 41], 4,
                     dict(qk_norm=True, plain_ctx_kv=True, gelu_ffn=True, rope_theta=500.0)),
    # long enough for the streaming attention kernel, grouped heads
    "bf16-streaming-gqa": (dict(name="v6", seed_id=106, A=1, m=1, H=64, d=512, n_heads=8, gamma=5,
                                n_layers=1, ff=512, dtype="bf16"), [20000], 2,
                           dict(qk_norm=True, rope_theta=10000.0)),
    # Eq 2 in one split with the fused row norm: the unnormalised context K/V
    # take 1 / rms(P) as their row scale
    "bf16-fused-plain": (dict(name="v7", seed_id=107, A=2, m=2, H=128, d=512, n_heads=4, gamma=5,
                              n_layers=1, ff=1024, dtype="bf16"), [20000, 12600], 2,
                         dict(qk_norm=True, plain_ctx_kv=True, rope_theta=10000.0)),
}


def _setup(case):
    kw, lengths, n_kv, sw = CASES[case]
    w = W.Workload(**kw, L=0)
    x = W.make_inputs(w, gains="random", lengths=lengths)
    x["layers"] = W.variant_layers(w, x["layers"], n_kv)
    dims = B.DsparkDims(m=w.m, H=w.H, d=w.d, n_heads=w.n_heads, gamma=w.gamma, n_layers=w.n_layers,
                        ff=w.ff, eps=w.eps, dtype=w.dtype, n_kv_heads=n_kv, **sw)
    u = Uploaded(w, x, device=DEV)
    return w, x, dims, u, n_kv, sw


def _oracle(w, x, n_kv, sw):
    return O.variant_forward(x["taps"], x["w_c"], x["ctx_norm"], x["cu"], x["block_in"], x["block_pos"],
                             x["layers"], x["out_norm"], w.n_heads, n_kv, w.eps,
                             ctx_norm_kv=not sw.get("plain_ctx_kv", False), qk_norm=sw.get("qk_norm", False),
                             theta=sw.get("rope_theta", 0.0),
                             act="gelu_tanh" if sw.get("gelu_ffn") else "silu")


@pytest.mark.parametrize("case", sorted(CASES))
def test_variant_forward_matches_oracle(case):
    w, x, dims, u, n_kv, sw = _setup(case)
    plan = B.plan_info(B.OP_BLOCK_FORWARD, dims, x["cu"])
    print(f"{case}: lengths {x['lengths'].tolist()} n_kv {n_kv} {sw} plan {plan}", flush=True)
    if "streaming" in case:
        assert plan["attn_streaming"] == 1
    if "fused" in case:
        assert plan["ctx_fused_norm"] == 1, plan
    out = B.block_forward(dims, u.cu, u.taps, u.w_c, u.ctx_norm, u.block_in, u.block_pos, u.layers,
                          u.out_norm, cu_dev=u.cu_dev)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    e = rel_err(got, _oracle(w, x, n_kv, sw))
    print(f"  forward rel err {e:.3e}")
    assert e < TOL[w.dtype]


@pytest.mark.parametrize("case", ["bf16-all", "f32-all-hd32"])
def test_variant_layer_matches_oracle(case):
    """One variant layer over a given H_ctx (dspark_block_layer)."""
    w, x, dims, u, n_kv, sw = _setup(case)
    C = O.ctx_fuse(x["taps"], x["w_c"], x["ctx_norm"], w.eps)
    C = W.bf16_round(C.astype(np.float32)) if w.dtype == "bf16" else C.astype(np.float32)
    D = O.block_init(x["block_in"], x["block_pos"]).astype(np.float32)
    h = torch.from_numpy(C).to(device=DEV, dtype=u.dt)
    out = B.block_layer(dims, u.cu, h, torch.from_numpy(D).to(DEV), u.layers[0], cu_dev=u.cu_dev)
    torch.cuda.synchronize()
    lw = x["layers"][0]
    Kc, Vc = O.variant_context_kv(C, x["cu"], lw, n_kv, w.eps, ctx_norm_kv=not sw.get("plain_ctx_kv", False),
                                  qk_norm=sw.get("qk_norm", False), theta=sw.get("rope_theta", 0.0))
    ref = O.variant_layer(Kc, Vc, x["cu"], D, lw, w.n_heads, n_kv, w.eps, qk_norm=sw.get("qk_norm", False),
                          theta=sw.get("rope_theta", 0.0), act="gelu_tanh" if sw.get("gelu_ffn") else "silu")
    e = rel_err(out.cpu().numpy(), ref)
    print(f"{case}: layer rel err {e:.3e}")
    assert e < TOL[w.dtype]


@pytest.mark.parametrize("case", ["bf16-all", "bf16-rope-gqa4"])
def test_variant_propose_over_cache_matches_oracle(case):
    """Appends in pieces (rotary positions continue from each sequence's
    length) and a propose, against the whole-context variant forward."""
    w, x, dims, u, n_kv, sw = _setup(case)
    cu = [int(c) for c in x["cu"]]
    cap = ((max(x["lengths"]) + 63) // 64) * 64 + 64
    cache = B.DraftCache(dims, w.A, cap, device=DEV)
    done = [0] * w.A
    for frac in (0.3, 0.31, 1.0):
        counts = [int(round(frac * (cu[b + 1] - cu[b]))) - done[b] for b in range(w.A)]
        idx = np.concatenate([np.arange(cu[b] + done[b], cu[b] + done[b] + counts[b]) for b in range(w.A)])
        taps = u.taps[:, torch.as_tensor(idx, device=DEV, dtype=torch.long)].contiguous()
        cache.append(taps, counts, u.w_c, u.ctx_norm, u.layers)
        done = [a + c for a, c in zip(done, counts)]
    out = cache.propose(u.block_in, u.block_pos, u.layers, u.out_norm)
    torch.cuda.synchronize()
    e = rel_err(out.cpu().numpy(), _oracle(w, x, n_kv, sw))
    print(f"{case}: propose over the cache rel err {e:.3e}")
    assert e < TOL[w.dtype]
