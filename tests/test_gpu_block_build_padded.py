"""Block construction (dspark_block_build, #buildBlock) and the padded-batch
forward with the key-padding mask (dspark_block_forward_padded, #maskBias)
against the oracle, through the C ABI."""
import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import TOL, Uploaded, dims_of, rel_err

torch = pytest.importorskip("torch")
B = pytest.importorskip("block_draft_context_amd")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"


def _f(a, t=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=t)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_block_build_matches_oracle(dtype):
    A, H, d, G = 5, 2560, 1024, 5
    bb = W.block_build_inputs(91, A=A, H=H, d=d, gamma=G, dtype=dtype)
    dims = B.DsparkDims(m=1, H=H, d=d, n_heads=8, gamma=G, n_layers=1, ff=2 * d, dtype=dtype)
    st = torch.bfloat16 if dtype == "bf16" else torch.float32
    got = B.block_build(dims, _f(bb["anchor_emb"]), _f(bb["tok_proj"].T, st), _f(bb["mask_emb"]))
    torch.cuda.synchronize()
    zero_pos = np.zeros((G, d))
    ref = O.build_block(bb["anchor_emb"], bb["tok_proj"], bb["mask_emb"], zero_pos)
    e = rel_err(got.cpu().numpy(), ref)
    print(f"{dtype}: block rows rel err {e:.2e}")
    assert e < 1e-5
    assert np.array_equal(got.cpu().numpy()[:, 1:], np.broadcast_to(bb["mask_emb"], (A, G - 1, d)))


def test_block_build_gamma1_and_into_the_forward():
    """gamma = 1 (the anchor row only), then a built block through the whole
    forward against #backbone (#buildBlock + layers + output norm)."""
    w = W.Workload("bb1", 92, A=2, m=2, H=128, d=256, n_heads=2, gamma=4, n_layers=2, ff=512,
                   dtype="bf16", L=0)
    x = W.make_inputs(w, gains="random", lengths=[300, 41])
    bb = W.block_build_inputs(92, A=2, H=w.H, d=w.d, gamma=w.gamma)
    u = Uploaded(w, x, device=DEV)
    dims = dims_of(B, w)
    d1 = B.DsparkDims(m=1, H=w.H, d=w.d, n_heads=2, gamma=1, n_layers=1, ff=512, dtype="bf16")
    one = B.block_build(d1, _f(bb["anchor_emb"]), _f(bb["tok_proj"].T, torch.bfloat16), None)
    bin_ = B.block_build(dims, _f(bb["anchor_emb"]), _f(bb["tok_proj"].T, torch.bfloat16), _f(bb["mask_emb"]))
    out = B.block_forward(dims, u.cu, u.taps, u.w_c, u.ctx_norm, bin_, u.block_pos, u.layers, u.out_norm,
                          cu_dev=u.cu_dev)
    torch.cuda.synchronize()
    assert np.array_equal(one.cpu().numpy()[:, 0], bin_.cpu().numpy()[:, 0])
    Hd = O.build_block(bb["anchor_emb"], bb["tok_proj"], bb["mask_emb"], x["block_pos"])
    ref = O.block_forward(x["taps"], x["w_c"], x["ctx_norm"], x["cu"], Hd, np.zeros_like(x["block_pos"]),
                          x["layers"], x["out_norm"], w.n_heads, w.eps)
    e = rel_err(out.cpu().numpy(), ref)
    print(f"built block through the forward: rel err {e:.2e}")
    assert e < TOL["bf16"]


PADDED = {
    # name: (workload kwargs, real lengths, L_ctx, placements)
    "bf16-mixed": (dict(name="p1", seed_id=93, A=3, m=2, H=128, d=256, n_heads=2, gamma=5, n_layers=2,
                        ff=512, dtype="bf16"), [420, 0, 300], 700, ["scatter", "lead", "lead"]),
    "f32-mixed": (dict(name="p2", seed_id=94, A=3, m=2, H=64, d=128, n_heads=4, gamma=3, n_layers=1,
                       ff=256, dtype="f32"), [50, 199, 0], 200, ["scatter", "scatter", "lead"]),
    # long enough for the streaming kernel; sequence 0 leaves a run of whole
    # 64-key blocks empty (masked) between its real rows
    "bf16-streaming-holes": (dict(name="p3", seed_id=95, A=2, m=1, H=64, d=256, n_heads=4, gamma=6,
                                  n_layers=1, ff=256, dtype="bf16"), [15000, 9000], 20000,
                             [np.concatenate([np.arange(0, 1000), np.arange(6000, 20000)]), "scatter"]),
}


@pytest.mark.parametrize("case", sorted(PADDED))
def test_padded_forward_matches_oracle(case):
    kw, lengths, L_ctx, placements = PADDED[case]
    w = W.Workload(**kw, L=0)
    x = W.make_inputs(w, gains="random", lengths=lengths)
    ptaps, mask = W.padded_layout(kw["seed_id"], x["taps"], x["cu"], L_ctx, placements, dtype=w.dtype)
    dims = dims_of(B, w)
    A = w.A
    plan = B.plan_info(B.OP_BLOCK_FORWARD, dims, [b * L_ctx for b in range(A + 1)])
    print(f"{case}: real lengths {lengths} of {L_ctx}, plan {plan}", flush=True)
    if "streaming" in case:
        assert plan["attn_streaming"] == 1
    u = Uploaded(w, x, device=DEV)
    st = u.dt
    taps_d = torch.stack([_f(t, st) for t in ptaps])
    out = B.block_forward_padded(dims, taps_d, L_ctx, _f(mask, torch.uint8), u.w_c, u.ctx_norm, u.block_in,
                                 u.block_pos, u.layers, u.out_norm)
    packed = B.block_forward(dims, u.cu, u.taps, u.w_c, u.ctx_norm, u.block_in, u.block_pos, u.layers,
                             u.out_norm, cu_dev=u.cu_dev)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    taps3 = [t.reshape(A, L_ctx, -1) for t in ptaps]
    ref = O.block_forward_padded(taps3, x["w_c"], x["ctx_norm"], mask, x["block_in"], x["block_pos"],
                                 x["layers"], x["out_norm"], w.n_heads, w.eps)
    e = rel_err(got, ref)
    ep = rel_err(got, packed.cpu().numpy())
    print(f"  padded vs oracle {e:.2e}, vs the packed forward of the real rows {ep:.2e}")
    assert e < TOL[w.dtype]
    assert ep < (5e-3 if w.dtype == "bf16" else 1e-5)
