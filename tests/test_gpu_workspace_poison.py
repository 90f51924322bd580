"""Every value a call reads from its workspace is written earlier in the same
call. Each entry point runs twice on the same inputs, once with a zeroed
workspace and once with a workspace of 0xFF bytes (a NaN in float32 and in
bfloat16): every output must be bitwise the same and finite. A kernel that
read a workspace value it had not written (a padding row, an empty tile's
partial, a stale split) would turn the second run's outputs into NaN or
change them."""
import numpy as np
import pytest

import workloads as W
from gpu_helpers import Uploaded, dims_of

torch = pytest.importorskip("torch")
B = pytest.importorskip("block_draft_context_amd")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]
DEV = "cuda:0"

# (workload kwargs, lengths): Eq 2 in several K splits, Eq 2 fused in one
# split (with and without a split last round), the streaming and head-split
# attention with empty sequences, float32, sixteen sequences
CASES = {
    "split-eq2": (dict(seed_id=201, A=2, m=4, H=256, d=256, n_heads=4, gamma=6, n_layers=2, ff=512,
                       dtype="bf16"), [1500, 700]),
    "fused-eq2-tail": (dict(seed_id=202, A=2, m=2, H=512, d=512, n_heads=4, gamma=5, n_layers=1,
                            ff=1024, dtype="bf16"), [20000, 13768]),
    "streaming-empty": (dict(seed_id=203, A=3, m=1, H=64, d=256, n_heads=2, gamma=3, n_layers=1, ff=512,
                             dtype="bf16"), [30011, 0, 11111]),
    "hsplit-ragged": (dict(seed_id=204, A=4, m=1, H=64, d=128, n_heads=4, gamma=1, n_layers=2, ff=384,
                           dtype="bf16"), [1, 65, 129, 0]),
    "f32": (dict(seed_id=205, A=3, m=2, H=128, d=128, n_heads=4, gamma=5, n_layers=2, ff=256,
                 dtype="f32"), [70, 0, 333]),
    "sixteen": (dict(seed_id=206, A=16, m=2, H=64, d=256, n_heads=2, gamma=5, n_layers=1, ff=1024,
                     dtype="bf16"), [37, 0, 250, 1, 64, 65, 300, 129, 7, 0, 200, 33, 128, 5, 90, 311]),
}


def _case(name):
    kw, lengths = CASES[name]
    w = W.Workload(name=name, L=0, **kw)
    x = W.make_inputs(w, gains="random", lengths=lengths)
    return w, x, Uploaded(w, x, device=DEV)


def _ws(need, poison):
    if poison:
        return torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    return torch.zeros(need, dtype=torch.uint8, device=DEV)


def _same(a, b, what):
    torch.cuda.synchronize()
    assert torch.isfinite(a.float()).all(), f"{what}: non-finite values with a NaN-filled workspace"
    assert torch.equal(a, b), f"{what}: differs between a zeroed and a NaN-filled workspace"


@pytest.mark.parametrize("case", sorted(CASES))
def test_forward_and_layer(case):
    w, x, u = _case(case)
    dims = dims_of(B, w)
    need = B.workspace_size(B.OP_BLOCK_FORWARD, dims, u.cu)
    outs, hs = [], []
    for poison in (False, True):
        h = torch.empty((x["T"], w.d), dtype=u.dt, device=DEV)
        o = B.block_forward(dims, u.cu, u.taps, u.w_c, u.ctx_norm, u.block_in, u.block_pos, u.layers,
                            u.out_norm, cu_dev=u.cu_dev, h_ctx_out=h, ws=_ws(need, poison))
        outs.append(o)
        hs.append(h)
    _same(outs[1], outs[0], "block_forward output")
    if x["T"] > 0:
        _same(hs[1], hs[0], "block_forward H_ctx")
    # one layer over that context, and Eq 2 alone
    need = B.workspace_size(B.OP_BLOCK_LAYER, dims, u.cu)
    d0 = (u.block_in + u.block_pos[None]).contiguous()
    lay = [B.block_layer(dims, u.cu, hs[0], d0, u.layers[0], cu_dev=u.cu_dev, ws=_ws(need, p))
           for p in (False, True)]
    _same(lay[1], lay[0], "block_layer output")
    if x["T"] > 0:
        need = B.workspace_size(B.OP_CTX_FUSE, dims, u.cu)
        hf = [B.ctx_fuse(dims, u.cu, u.taps, u.w_c, u.ctx_norm, cu_dev=u.cu_dev, ws=_ws(need, p))
              for p in (False, True)]
        _same(hf[1], hf[0], "ctx_fuse H_ctx")


@pytest.mark.parametrize("case", ["split-eq2", "fused-eq2-tail", "sixteen"])
def test_cache_append_and_propose(case):
    w, x, u = _case(case)
    dims = dims_of(B, w)
    Ls = [int(x["cu"][b + 1] - x["cu"][b]) for b in range(w.A)]
    cap = ((max(Ls) + 63) // 64) * 64
    results = []
    for poison in (False, True):
        cache = B.DraftCache(dims, w.A, cap, device=DEV)
        need = B.workspace_size(B.OP_CTX_APPEND, dims, x["cu"])
        cache.append(u.taps, Ls, u.w_c, u.ctx_norm, u.layers, ws=_ws(need, poison))
        need = B.workspace_size(B.OP_BLOCK_PROPOSE, dims, cache.cu())
        out = cache.propose(u.block_in, u.block_pos, u.layers, u.out_norm, ws=_ws(need, poison))
        results.append((cache.buf.clone(), out))
    _same(results[1][1], results[0][1], "propose output")
    assert torch.equal(results[1][0], results[0][0]), "cache contents differ"


def test_padded_forward():
    w, x, u = _case("split-eq2")
    dims = dims_of(B, w)
    L_ctx = 1600
    taps, mask = W.padded_layout(207, x["taps"], x["cu"], L_ctx, ["scatter", "lead"], dtype=w.dtype)
    dt = u.dt
    td = torch.stack([torch.from_numpy(np.ascontiguousarray(t)).to(device=DEV, dtype=dt) for t in taps])
    md = torch.from_numpy(mask).to(DEV)
    need = B.padded_workspace_size(dims, w.A, L_ctx)
    outs = [B.block_forward_padded(dims, td, L_ctx, md, u.w_c, u.ctx_norm, u.block_in, u.block_pos, u.layers,
                                   u.out_norm, ws=_ws(need, p)) for p in (False, True)]
    _same(outs[1], outs[0], "padded forward output")


def test_markov_draft():
    A, G, d, V, r = 17, 5, 256, 5000, 256
    x = W.markov_inputs(208, A=A, gamma=G, d=d, vocab=V, rank=r)
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=t)
    g = dict(block=f(x["block"]), U=f(x["base_logits"]), anchor=f(x["anchor"], torch.int32),
             w1=f(x["w1"], torch.bfloat16), w2=f(x["w2"], torch.bfloat16), cw=f(x["conf_w"]), cb=f(x["conf_b"]))
    dims = B.DsparkDims(m=1, H=64, d=d, n_heads=1, gamma=G, n_layers=1, ff=128, dtype="bf16")
    need = B.markov_workspace_size(dims, A, V, r)
    res = [B.markov_draft(dims, g["block"], g["U"], g["anchor"], g["w1"], g["w2"], g["cw"], g["cb"],
                          ws=_ws(need, p)) for p in (False, True)]
    for k, what in enumerate(("tokens", "confidence", "draft logits")):
        _same(res[1][k], res[0][k], f"markov {what}")
