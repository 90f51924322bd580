"""The Markov head, confidence head and greedy draft loop (dspark_markov_draft)
against the oracle's markov_draft, through the C ABI.

Tokens: where floating point decides an integer, both sides decide on the
float32 logits (the compute type of module-dflash.ts); the kernels and the
oracle sum in different orders, so each drafted position is checked along
the GPU's own token chain (teacher forcing): the oracle's float64 logits of
that position, given the GPU's previous token, must put the GPU's token
within the float32 summation bound of the maximum, and every position whose
top-two margin exceeds that bound must pick the oracle's token exactly.
Where all margins exceed the bound the whole token array equals the
oracle's free-running draft. Ties (exactly equal logits) go to the lowest
index on both sides."""
import numpy as np
import pytest

import oracle as O
import workloads as W

torch = pytest.importorskip("torch")
B = pytest.importorskip("block_draft_context_amd")
pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda:0"


def _upload(x, dtype):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=t)
    return dict(block=f(x["block"]), U=f(x["base_logits"]), anchor=f(x["anchor"], torch.int32),
                w1=f(x["w1"], dt), w2=f(x["w2"], dt), cw=f(x["conf_w"]), cb=f(x["conf_b"]))


def _dims(d, gamma, dtype):
    return B.DsparkDims(m=1, H=64, d=d, n_heads=1, gamma=gamma, n_layers=1, ff=128, dtype=dtype)


def _run(x, d, gamma, dtype):
    g = _upload(x, dtype)
    toks, conf, logits = B.markov_draft(_dims(d, gamma, dtype), g["block"], g["U"], g["anchor"], g["w1"],
                                        g["w2"], g["cw"], g["cb"])
    torch.cuda.synchronize()
    return toks.cpu().numpy(), conf.cpu().numpy(), logits.cpu().numpy()


def _teacher_forced(x, toks):
    """Oracle float64 logits and confidences of every position given the
    GPU's previous tokens, and the float32 summation bound of each logit."""
    A, G, d = x["block"].shape
    w1 = x["w1"].astype(np.float64)
    w2 = x["w2"].astype(np.float64)          # [vocab, rank]
    r = w1.shape[1]
    u = 2.0 ** -24
    logits = np.zeros(x["base_logits"].shape)
    bound = np.zeros((A, G))
    conf = np.zeros((A, G))
    for b in range(A):
        prev = int(x["anchor"][b])
        for k in range(G):
            e1 = w1[prev]
            lk = x["base_logits"][b, k].astype(np.float64) + w2 @ e1
            logits[b, k] = lk
            mag = np.abs(w2) @ np.abs(e1) + np.abs(x["base_logits"][b, k])
            bound[b, k] = 2.0 * (r + 2) * u * float(mag.max())
            z = x["block"][b, k] @ x["conf_w"][:d] + e1 @ x["conf_w"][d:] + x["conf_b"][0]
            conf[b, k] = 1.0 / (1.0 + np.exp(-z))
            prev = int(toks[b, k])
    return logits, conf, bound


def _check(x, d, G, dtype, toks, conf, logits):
    ol, oc, bound = _teacher_forced(x, toks)
    top2 = np.sort(ol, axis=-1)[..., -2:]
    margin = top2[..., 1] - top2[..., 0]
    chosen = np.take_along_axis(ol, toks[..., None].astype(np.int64), axis=-1)[..., 0]
    assert np.all(chosen >= ol.max(axis=-1) - bound), "a token outside the float32 bound of the maximum"
    decided = margin > bound
    assert np.array_equal(toks[decided], np.argmax(ol, axis=-1)[decided])
    print(f"{dtype}: margins min {margin.min():.3e}, bound max {bound.max():.3e}, "
          f"{int(decided.sum())}/{decided.size} positions decided beyond the bound")
    if decided.all():
        ot, _, _ = O.markov_draft(x["block"], x["base_logits"], x["anchor"], x["w1"], x["w2"].T,
                                  x["conf_w"], float(x["conf_b"][0]))
        assert np.array_equal(toks, ot), "free-running draft differs from the oracle"
    assert np.max(np.abs(conf - oc)) < 1e-4
    el = float(np.max(np.abs(logits - ol)) / np.max(np.abs(ol)))
    print(f"  confidence max abs err {np.max(np.abs(conf - oc)):.2e}, draft logits rel err {el:.2e}")
    assert el < 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_markov_draft_matches_oracle(dtype):
    A, G, d, V, r = 5, 6, 256, 5000, 128
    x = W.markov_inputs(81 if dtype == "bf16" else 82, A=A, gamma=G, d=d, vocab=V, rank=r, dtype=dtype)
    _check(x, d, G, dtype, *_run(x, d, G, dtype))


# (A, gamma, vocab, rank): more than 16 sequences (two sequence groups of the
# matrix-core step kernel), every rank class it instantiates up to 512
# with ragged last vocabulary chunks, ranks above 512 (the row-GEMM path),
# the measured size (1 and 16 sequences, vocabulary 131072, rank 256) and a
# one-position block
SHAPES = [(20, 5, 5000, 256), (3, 4, 4104, 512), (17, 3, 3000, 192), (1, 5, 2056, 64),
          (2, 2, 1000, 576), (33, 2, 808, 320), (16, 5, 131072, 256), (1, 5, 131072, 256),
          (4, 1, 1000, 128)]


@pytest.mark.parametrize("A,G,V,r", SHAPES, ids=[f"A{a}-g{g}-V{v}-r{r}" for a, g, v, r in SHAPES])
def test_markov_draft_shapes(A, G, V, r):
    d = 128
    x = W.markov_inputs(85 + r, A=A, gamma=G, d=d, vocab=V, rank=r)
    _check(x, d, G, "bf16", *_run(x, d, G, "bf16"))


def test_markov_ties_and_closed_forms():
    """w2 = 0 (initFromDims's start): tokens are the argmax of the base
    logits, exact ties resolved to the lowest index; conf_w = 0, conf_b = 0
    give confidence 1/2 exactly."""
    A, G, d, V, r = 3, 4, 128, 2048, 64
    x = W.markov_inputs(83, A=A, gamma=G, d=d, vocab=V, rank=r, zero_w2=True)
    U = x["base_logits"]
    U[0, :, 1500] = U[0, :, 700] = 50.0         # equal maxima: the lower index wins
    U[1, 2, :] = 3.0                            # all equal: index 0
    U[2, 1, 2047] = 60.0
    x["conf_w"][:] = 0.0
    x["conf_b"][:] = 0.0
    toks, conf, logits = _run(x, d, G, "bf16")
    assert np.array_equal(logits, U)
    assert np.array_equal(toks, np.argmax(U, axis=-1))
    assert np.all(toks[0] == 700) and toks[1, 2] == 0 and toks[2, 1] == 2047
    assert np.all(conf == 0.5)


def test_markov_chain_feeds_back():
    """Zero base logits, one-hot Markov embeddings (w1 = I, rank = vocab)
    and w2 the shift v -> v + 1: the greedy draft counts up from the anchor."""
    A, G, d, V = 4, 7, 128, 64
    x = W.markov_inputs(84, A=A, gamma=G, d=d, vocab=V, rank=V)
    x["base_logits"][:] = 0.0
    x["w1"] = np.eye(V, dtype=np.float32)
    x["w2"] = np.roll(np.eye(V, dtype=np.float32), 1, axis=0)   # [vocab, rank]: row v+1 picks column v
    x["anchor"] = np.array([0, 5, 62, 63], dtype=np.int32)
    toks, _, _ = _run(x, d, G, "bf16")
    want = (x["anchor"][:, None] + np.arange(1, G + 1)[None, :]) % V
    assert np.array_equal(toks, want), (toks, want)
