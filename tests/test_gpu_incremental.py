"""The incremental context (dspark_ctx_append + dspark_block_propose over a
draft cache) against the oracle, through the C ABI.

The oracle side is its own cache (oracle.cache_append / block_propose) and
its full recompute (oracle.block_forward over the whole context), which the
oracle pins show equal. The cache is decoded on the host with the layout
include/dspark.h documents: the K/V rows of every appended position are
compared with the oracle's, and every row not yet appended must still hold
exact zeros (rows land at exactly their offsets)."""
import ctypes

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import TOL, Uploaded, dims_of, rel_err

torch = pytest.importorskip("torch")
B = pytest.importorskip("block_draft_context_amd")
from block_draft_context_amd import _lib as L  # noqa: E402

gpu = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def decode_cache(raw: np.ndarray, w, A: int, cap: int):
    """K, V as float64 arrays [n_layers, A, cap, d] from the cache bytes."""
    esz = 2 if w.dtype == "bf16" else 4
    if esz == 2:
        vals = (raw.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    else:
        vals = raw.view(np.float32)
    hd, nh = w.head_dim, w.n_heads
    E = 16 // esz
    R, KG = E // 2, 128 // hd
    slab = A * cap
    vals = vals.reshape(w.n_layers, 2, nh, slab * hd)
    t = np.arange(slab)[:, None]
    c = np.arange(hd)[None, :]
    k_off = ((t >> 6) * (hd // E) + c // E) * (64 * E) + (t & 63) * E + c % E
    kk = t & 63
    vec = (kk // (KG * R)) * 64 + ((kk // R) % KG) * (hd // 2) + c // 2
    v_off = (t >> 6) * 64 * hd + vec * E + (kk % R) * 2 + (c & 1)
    K = vals[:, 0][:, :, k_off]      # [layers, heads, slab, hd]
    V = vals[:, 1][:, :, v_off]
    K = K.transpose(0, 2, 1, 3).reshape(w.n_layers, A, cap, nh * hd)
    V = V.transpose(0, 2, 1, 3).reshape(w.n_layers, A, cap, nh * hd)
    return K.astype(np.float64), V.astype(np.float64)


def _workload(seed_id, final_lengths, **kw):
    base = dict(name=f"inc{seed_id}", seed_id=seed_id, A=len(final_lengths), m=2, H=128, d=256,
                n_heads=2, gamma=5, n_layers=2, ff=512, dtype="bf16", L=0)
    base.update(kw)
    w = W.Workload(**base)
    return w, W.make_inputs(w, gains="random", lengths=final_lengths)


def _pieces_taps(x, pieces, done, device, dt):
    """Device taps of one append: the next counts[b] rows of each sequence."""
    cu = [int(c) for c in x["cu"]]
    rows = []
    for b, n in enumerate(pieces):
        r0 = cu[b] + done[b]
        rows.append(np.arange(r0, r0 + n))
    idx = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    taps = torch.empty((len(x["taps"]), len(idx), x["taps"][0].shape[1]), dtype=dt, device=device)
    for j, t in enumerate(x["taps"]):
        taps[j].copy_(torch.from_numpy(np.ascontiguousarray(t[idx])).to(device=device, dtype=dt))
    return taps, [t[idx] for t in x["taps"]]


def _run(w, x, cap, schedule, *, check_every=False):
    dev = "cuda:0"
    u = Uploaded(w, x, device=dev)
    dims = dims_of(B, w)
    cache = B.DraftCache(dims, w.A, cap, device=dev)
    ocache = O.DraftCache(w.A, w.n_layers, w.d)
    done = [0] * w.A
    results = []
    for step, counts in enumerate(schedule):
        taps, taps_np = _pieces_taps(x, counts, done, dev, u.dt)
        cache.append(taps, counts, u.w_c, u.ctx_norm, u.layers)
        ncu = np.concatenate([[0], np.cumsum(counts)])
        O.cache_append(ocache, taps_np, ncu, x["w_c"], x["ctx_norm"], x["layers"], w.eps)
        done = [a + c for a, c in zip(done, counts)]
        if check_every or step == len(schedule) - 1:
            plan = B.plan_info(B.OP_BLOCK_PROPOSE, dims, cache.cu())
            out = cache.propose(u.block_in, u.block_pos, u.layers, u.out_norm)
            torch.cuda.synchronize()
            ref = O.block_propose(ocache, x["block_in"], x["block_pos"], x["layers"], x["out_norm"],
                                  w.n_heads, w.eps)
            e = rel_err(out.cpu().numpy(), ref)
            print(f"  after append {step} lengths={cache.lengths} plan={plan}: propose rel err {e:.3e}",
                  flush=True)
            assert np.all(np.isfinite(out.cpu().numpy()))
            assert e < TOL[w.dtype]
            results.append(out)
    assert cache.lengths == done
    return cache, ocache, u, results


def _check_cache(w, cache, ocache):
    torch.cuda.synchronize()
    K, V = decode_cache(cache.buf.cpu().numpy(), w, cache.A, cache.cap)
    for b in range(cache.A):
        n = cache.lengths[b]
        # rows never appended: untouched, still the zeros of the reset
        assert np.all(K[:, b, n:] == 0.0) and np.all(V[:, b, n:] == 0.0), b
        for i in range(w.n_layers):
            if n == 0:
                continue
            ek = rel_err(K[i, b, :n], ocache.K[b][i])
            ev = rel_err(V[i, b, :n], ocache.V[b][i])
            assert ek < TOL[w.dtype] and ev < TOL[w.dtype], (b, i, ek, ev)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_appends_then_propose_match_oracle(dtype):
    """Appends of every size (empty, single rows at unaligned positions, and
    more than 512 rows, which takes the big-tile K/V product), proposing
    after each; then the cache contents row by row."""
    kw = {} if dtype == "bf16" else dict(d=128, n_heads=4, ff=256)
    w, x = _workload(71 if dtype == "bf16" else 72, [2600, 0, 1500], dtype=dtype, **kw)
    sched = [[700, 0, 3], [1, 0, 1], [0, 0, 0], [1200, 0, 900], [699, 0, 596]]
    print(f"{dtype}: schedule {sched}")
    cache, ocache, u, _ = _run(w, x, 4096, sched, check_every=True)
    _check_cache(w, cache, ocache)


@pytest.mark.parametrize("dtype", ["bf16"])
def test_incremental_equals_full_forward(dtype):
    """The same context appended in pieces or given whole to
    dspark_block_forward: the same draft block up to the bf16 roundings of
    H_ctx and K/V (a single forward may split its Eq 2 product differently)."""
    w, x = _workload(73, [3000, 517], n_layers=3)
    cache, ocache, u, res = _run(w, x, 3072, [[1000, 17], [2000, 500]])
    full = B.block_forward(dims_of(B, w), u.cu, u.taps, u.w_c, u.ctx_norm, u.block_in, u.block_pos,
                           u.layers, u.out_norm, cu_dev=u.cu_dev)
    torch.cuda.synchronize()
    e = rel_err(res[-1].cpu().numpy(), full.cpu().numpy())
    print(f"  incremental vs full forward rel diff {e:.3e}")
    assert e < 5e-3
    _check_cache(w, cache, ocache)


def test_streaming_attention_over_the_cache():
    """A long cached context takes the streaming split-K kernel, whose tiles
    address sequence b at b * cap."""
    w, x = _workload(74, [20000, 9000], d=256, n_heads=4, gamma=6, n_layers=1)
    dims = dims_of(B, w)
    p = B.plan_info(B.OP_BLOCK_PROPOSE, dims, [0, 20000, 29000])
    assert p["attn_streaming"] == 1, p
    cache, ocache, u, _ = _run(w, x, 20032, [[12000, 4000], [8000, 5000]])
    _check_cache(w, cache, ocache)


def test_fused_eq2_append():
    """An append large enough for Eq 2 in one split with the row norm folded
    into the K/V row scale (the fused epilogue writes Y = P * ctx_norm and
    row sums; no H_ctx is stored), then a small split-K append."""
    w, x = _workload(75, [20000, 13000], d=512, n_heads=4, gamma=5, n_layers=1)
    dims = dims_of(B, w)
    assert B.plan_info(B.OP_CTX_APPEND, dims, [0, 20000, 32600])["ctx_fused_norm"] == 1
    assert B.plan_info(B.OP_CTX_APPEND, dims, [0, 0, 400])["ctx_fused_norm"] == 0
    cache, ocache, u, _ = _run(w, x, 20032, [[20000, 12600], [0, 400]], check_every=True)
    _check_cache(w, cache, ocache)


for _name in ("test_appends_then_propose_match_oracle", "test_incremental_equals_full_forward",
              "test_streaming_attention_over_the_cache", "test_fused_eq2_append"):
    for _m in gpu:
        globals()[_name] = _m(globals()[_name])


def test_append_rejects_overflow_before_launching():
    """pos + new rows beyond cap: DSPARK_EINVAL before anything is enqueued
    (host-only check; the pointers are never touched)."""
    dm = L.Dims(2, 128, 256, 2, 5, 2, 512, 1e-6, L.BF16)
    A, cap = 2, 128
    ncu = (ctypes.c_int32 * 3)(0, 100, 140)
    pos = (ctypes.c_int32 * 2)(0, 100)     # sequence 1: 100 + 40 > 128
    taps = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    lws = (L.LayerWeights * 2)(*[L.LayerWeights(*([0x1000] * 9))] * 2)
    st = L.lib().dspark_ctx_append(ctypes.byref(dm), A, cap, ncu, 0x2000, pos, 0x2000, taps, 128,
                                   0x3000, 0x4000, lws, 0x5000, 0x6000, 1 << 40, None)
    assert st == L.EINVAL and "do not fit" in L.lib().dspark_last_error().decode()
    assert L.lib().dspark_cache_bytes(ctypes.byref(dm), 2, 100) == 0    # cap not a multiple of 64
    assert L.lib().dspark_cache_bytes(ctypes.byref(dm), 2, 128) == 2 * 2 * 2 * 128 * 256 * 2
    cu = (ctypes.c_int32 * 3)(0, 129, 129)
    st = L.lib().dspark_block_propose(ctypes.byref(dm), A, cap, cu, 0x2000, 0x5000, 0x3000, 0x3000,
                                      lws, None, 0x3000, 0x6000, 1 << 40, None)
    assert st == L.EINVAL and "cached rows" in L.lib().dspark_last_error().decode()
