"""The no-allocation entry point (dspark_block_layer_noalloc) against the
workspace entry point (dspark_block_layer) it is a variant of, through the C
ABI: two calls in a row on the library's device scratch, the second with a
smaller input, each compared with the workspace path and with the oracle."""
import ctypes

import numpy as np
import pytest

import oracle as O
import workloads as W
from gpu_helpers import TOL, Uploaded, dims_of, rel_err

torch = pytest.importorskip("torch")
B = pytest.importorskip("block_draft_context_amd")
from block_draft_context_amd import _lib as L  # noqa: E402


def _case(seed_id, lengths, **kw):
    base = dict(name=f"na{seed_id}", seed_id=seed_id, A=len(lengths), m=2, H=128, d=256, n_heads=2,
                gamma=5, n_layers=1, ff=512, dtype="bf16", L=0)
    base.update(kw)
    w = W.Workload(**base)
    return w, W.make_inputs(w, gains="random", lengths=lengths)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    """Checked on the host before anything is enqueued (no device call)."""
    dm = L.Dims(1, 64, 1024, 8, 5, 1, 2048, 1e-6, L.BF16)
    cu = (ctypes.c_int32 * 2)(0, 40000)
    lw = L.LayerWeights(*([0x1000] * 9))
    st = L.lib().dspark_block_layer_noalloc(ctypes.byref(dm), 1, cu, 0x2000, 0x3000, 0x4000, 0x4000,
                                            ctypes.byref(lw), None)
    assert st == L.EUNSUPPORTED
    assert "at most" in L.lib().dspark_last_error().decode()


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
def test_noalloc_matches_workspace_entry_point():
    dev = "cuda:0"
    cases = [_case(61, [3000, 0, 1400], gamma=6),          # the larger call first
             _case(62, [500, 37], d=128, n_heads=4, gamma=3)]   # then a smaller one
    for w, x in cases:
        dims = dims_of(B, w)
        need = B.workspace_size(B.OP_BLOCK_LAYER, dims, x["cu"])
        assert need <= L.NOALLOC_SCRATCH_BYTES
        u = Uploaded(w, x, device=dev)
        C = O.ctx_fuse(x["taps"], x["w_c"], x["ctx_norm"], w.eps)
        C = W.bf16_round(C.astype(np.float32))
        D = O.block_init(x["block_in"], x["block_pos"]).astype(np.float32)
        h = torch.from_numpy(C).to(device=dev, dtype=u.dt)
        d_in = torch.from_numpy(D).to(dev)
        ref = B.block_layer(dims, u.cu, h, d_in, u.layers[0], cu_dev=u.cu_dev)
        out = torch.full_like(d_in, float("nan"))
        B.block_layer_noalloc(dims, u.cu, h, d_in, u.layers[0], cu_dev=u.cu_dev, d_out=out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got))
        # the same kernels on the same inputs: bitwise the same rows
        e_ws = rel_err(got, ref.cpu().numpy())
        assert np.array_equal(got, ref.cpu().numpy())
        e_or = rel_err(got, O.block_layer(C, x["cu"], D, x["layers"][0], w.n_heads, w.eps))
        print(f"{w.name}: lengths={x['lengths'].tolist()} vs workspace path {e_ws:.2e}, vs oracle {e_or:.2e}")
        assert e_ws < 1e-6
        assert e_or < TOL[w.dtype]
