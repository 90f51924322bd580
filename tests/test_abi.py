"""C ABI contract on the host: the library loads, exports every function that
include/dspark.h declares, sizes workspaces, and rejects bad arguments with
the documented status before touching the GPU (these calls never reach a
HIP API)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dspark.h")


@pytest.fixture(scope="module")
def L():
    from block_draft_context_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from block_draft_context_amd.build import build
        build()
    return _lib


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("dspark_ctx_fuse", "dspark_block_layer", "dspark_block_forward",
              "dspark_workspace_size", "dspark_last_error"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    lib = L.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (dspark_\w+)", out))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(lib, n), n
    assert sorted(L.EXPORTS) == declared_functions()


def test_version_and_kernel_names(L):
    import block_draft_context_amd as B
    assert "gfx950" in B.version()
    names = B.kernel_names()
    assert "attn_split_k" in names and "gemm_ctx_kv" in names and len(set(names)) == len(names)


def _dims(L, **kw):
    base = dict(m=4, H=2560, d=1024, n_heads=8, gamma=5, n_layers=5, ff=2048, eps=1e-6, dtype=1)
    base.update(kw)
    return L.Dims(**base)


def _cu(vals):
    return (ctypes.c_int32 * len(vals))(*vals)


def test_workspace_size_grows_with_context(L):
    lib = L.lib()
    dm = _dims(L)
    sizes = [lib.dspark_workspace_size(L.OP_BLOCK_FORWARD, ctypes.byref(dm), 1, _cu([0, T]))
             for T in (0, 64, 2048, 131072)]
    assert all(s > 0 for s in sizes)
    assert sizes == sorted(sizes)
    # K/V of 5 layers for 131072 rows in bf16 alone is 2.5 GiB
    assert sizes[-1] >= 5 * 2 * 131072 * 1024 * 2
    one = lib.dspark_workspace_size(L.OP_BLOCK_LAYER, ctypes.byref(dm), 1, _cu([0, 131072]))
    assert one < sizes[-1]


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d=1000), 2, "head_dim"),
    (dict(n_heads=3), 1, "not divisible"),
    (dict(gamma=0), 1, "positive"),
    (dict(gamma=17), 2, "gamma"),
    (dict(dtype=7), 2, "dtype"),
    (dict(H=100), 2, "multiple of 64"),
    (dict(ff=100), 2, "multiple of 128"),
    (dict(ff=16384), 2, "16256"),
    (dict(n_layers=0), 1, "n_layers"),
    (dict(eps=-1.0), 1, "eps"),
])
def test_bad_dims_are_rejected(L, kw, status, msg):
    lib = L.lib()
    dm = _dims(L, **kw)
    assert lib.dspark_workspace_size(L.OP_BLOCK_FORWARD, ctypes.byref(dm), 1, _cu([0, 8])) == 0
    assert msg in lib.dspark_last_error().decode()
    taps = (ctypes.c_void_p * 4)(*[0x1000] * 4)
    st = lib.dspark_block_forward(ctypes.byref(dm), 1, _cu([0, 8]), 0x2000, taps, 2560, 0x3000, 0x4000,
                                  0x5000, 0x6000, None, None, None, 0x7000, 0x8000, 1 << 40, None)
    assert st == status


@pytest.mark.parametrize("cu,msg", [([1, 8], "cu[0]"), ([0, 8, 4], "decreasing")])
def test_bad_offsets_are_rejected(L, cu, msg):
    lib = L.lib()
    dm = _dims(L)
    A = len(cu) - 1
    assert lib.dspark_workspace_size(L.OP_CTX_FUSE, ctypes.byref(dm), A, _cu(cu)) == 0
    assert msg in lib.dspark_last_error().decode()


def test_entry_points_check_pointers_and_workspace(L):
    lib = L.lib()
    dm = _dims(L)
    cu = _cu([0, 128])
    taps = (ctypes.c_void_p * 4)(*[0x1000] * 4)
    need = lib.dspark_workspace_size(L.OP_CTX_FUSE, ctypes.byref(dm), 1, cu)
    # workspace too small
    st = lib.dspark_ctx_fuse(ctypes.byref(dm), 1, cu, 0x2000, taps, 2560, 0x3000, 0x4000, 0x5000,
                             0x6000, need - 1, None)
    assert st == L.EWORKSPACE and "workspace" in lib.dspark_last_error().decode()
    # misaligned output
    st = lib.dspark_ctx_fuse(ctypes.byref(dm), 1, cu, 0x2000, taps, 2560, 0x3000, 0x4000, 0x5004,
                             0x6000, need, None)
    assert st == L.EINVAL and "aligned" in lib.dspark_last_error().decode()
    # ld_tap below H
    st = lib.dspark_ctx_fuse(ctypes.byref(dm), 1, cu, 0x2000, taps, 2048, 0x3000, 0x4000, 0x5000,
                             0x6000, need, None)
    assert st == L.EINVAL and "ld_tap" in lib.dspark_last_error().decode()
    # NULL tap
    taps0 = (ctypes.c_void_p * 4)(0x1000, None, 0x1000, 0x1000)
    st = lib.dspark_ctx_fuse(ctypes.byref(dm), 1, cu, 0x2000, taps0, 2560, 0x3000, 0x4000, 0x5000,
                             0x6000, need, None)
    assert st == L.EINVAL and "taps[1]" in lib.dspark_last_error().decode()
    # NULL layer weight
    lw = L.LayerWeights(0x1000, 0x1000, None, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000)
    need_l = lib.dspark_workspace_size(L.OP_BLOCK_LAYER, ctypes.byref(dm), 1, cu)
    st = lib.dspark_block_layer(ctypes.byref(dm), 1, cu, 0x2000, 0x3000, 0x4000, 0x4000,
                                ctypes.byref(lw), 0x6000, need_l, None)
    assert st == L.EINVAL and "wk" in lib.dspark_last_error().decode()
    # too many block rows
    st = lib.dspark_block_layer(ctypes.byref(dm), 300, _cu([0] * 301), 0x2000, 0x3000, 0x4000,
                                0x4000, ctypes.byref(lw), 0x6000, need_l, None)
    assert st == L.EUNSUPPORTED


def test_taps_over_4gib_are_rejected(L):
    """The projection kernels address a tap with 32-bit byte offsets."""
    lib = L.lib()
    dm = _dims(L)
    T = 900000                                   # 900000 * 2560 * 2 bytes > 4 GiB
    cu = _cu([0, T])
    taps = (ctypes.c_void_p * 4)(*[0x1000] * 4)
    st = lib.dspark_ctx_fuse(ctypes.byref(dm), 1, cu, 0x2000, taps, 2560, 0x3000, 0x4000, 0x5000,
                             0x6000, 1 << 50, None)
    assert st == L.EUNSUPPORTED and "4 GiB" in lib.dspark_last_error().decode()


def test_h_ctx_and_w_c_over_4gib_are_rejected(L):
    """The context projections address H_ctx and W_c with 32-bit byte
    offsets; an H_ctx or W_c of 4 GiB or more is refused before anything
    runs, also where every tap is small."""
    lib = L.lib()
    # H = 64, d = 2048: the taps span 1.1e6 * 64 * 2 bytes, H_ctx 1.1e6 * 2048 * 2 > 4 GiB
    dm = L.Dims(1, 64, 2048, 16, 5, 1, 4096, 1e-6, L.BF16)
    T = 1100000
    cu = _cu([0, T])
    lw = L.LayerWeights(*([0x1000] * 9))
    st = lib.dspark_block_layer(ctypes.byref(dm), 1, cu, 0x2000, 0x3000, 0x4000, 0x4000,
                                ctypes.byref(lw), 0x6000, 1 << 50, None)
    assert st == L.EUNSUPPORTED and "H_ctx" in lib.dspark_last_error().decode()
    taps = (ctypes.c_void_p * 1)(0x1000)
    st = lib.dspark_ctx_fuse(ctypes.byref(dm), 1, cu, 0x2000, taps, 64, 0x3000, 0x4000, 0x5000,
                             0x6000, 1 << 50, None)
    assert st == L.EUNSUPPORTED and "H_ctx" in lib.dspark_last_error().decode()
    assert lib.dspark_workspace_size(L.OP_BLOCK_LAYER, ctypes.byref(dm), 1, cu) == 0
    # W_c = d * m * H = 2048 * 16 * 65536 bf16 elements = 4 GiB, over 64 rows of context
    dm = L.Dims(16, 65536, 2048, 16, 5, 1, 4096, 1e-6, L.BF16)
    cu = _cu([0, 64])
    taps = (ctypes.c_void_p * 16)(*[0x1000] * 16)
    st = lib.dspark_ctx_fuse(ctypes.byref(dm), 1, cu, 0x2000, taps, 65536, 0x3000, 0x4000, 0x5000,
                             0x6000, 1 << 50, None)
    assert st == L.EUNSUPPORTED and "W_c" in lib.dspark_last_error().decode()
    # the same sizes are fine for a layer, which does not read W_c
    assert lib.dspark_workspace_size(L.OP_BLOCK_LAYER, ctypes.byref(dm), 1, cu) > 0


def test_python_binding_raises_with_message(L):
    import block_draft_context_amd as B
    with pytest.raises(B.DsparkError) as e:
        B.workspace_size(B.OP_BLOCK_FORWARD, B.DsparkDims(m=2, H=64, d=128, n_heads=3, gamma=2,
                                                          n_layers=1, ff=128), [0, 4])
    assert "not divisible" in str(e.value)


def _plan(L, op, dm, cu):
    k = len(L.PLAN_FIELDS)
    out = (ctypes.c_int64 * k)()
    n = L.lib().dspark_plan_info(op, ctypes.byref(dm), len(cu) - 1, _cu(cu), out, k)
    assert n == k, L.lib().dspark_last_error().decode()
    return dict(zip(L.PLAN_FIELDS, list(out)))


def test_ctx_splits_cover_every_column(L):
    """The Eq 2 projection's K splits cover all m*H columns with no empty
    split, for every storage type and kernel choice (K / splits need not be
    whole: e.g. float32 m=3, H=2304 once split 43 ways at 160 columns left 32
    columns out)."""
    checked = 0
    for dtype in (L.F32, L.BF16):
        for m in (1, 2, 3, 4, 5, 7, 16):
            for H in (64, 192, 2304, 2560, 3584, 5568):
                for d in (128, 384, 768, 1024, 2048):
                    for T in (1, 64, 100, 511, 512, 2048, 9000, 131072):
                        dm = _dims(L, m=m, H=H, d=d, n_heads=d // 128, dtype=dtype)
                        if d * m * H * (2 if dtype == L.BF16 else 4) >= 1 << 32:
                            continue
                        p = _plan(L, L.OP_CTX_FUSE, dm, [0, T])
                        K = m * H
                        s, kps = p["ctx_splits"], p["ctx_k_per_split"]
                        bk = 16 if dtype == L.F32 else 64
                        assert s >= 1 and kps % bk == 0, (dtype, m, H, d, T, p)
                        assert s * kps >= K and (s - 1) * kps < K, (dtype, m, H, d, T, p)
                        checked += 1
    assert checked > 1000


def test_plan_fuses_the_eq2_norm_in_one_split(L):
    """Eq 2 takes the fused epilogue (bf16 Y rows and row sums, the row norm
    folded into the K/V row scale) exactly when it runs as one K split on
    the big-tile kernel: bf16, d a multiple of 256, at least 512 rows and
    enough 256x256 tiles to fill the chip; ops without Eq 2 never do."""
    for dtype in (L.F32, L.BF16):
        for d in (128, 768, 1024, 2048):
            for T in (64, 2048, 8192, 16128, 16129, 131072):
                dm = _dims(L, m=4, H=2560, d=d, n_heads=d // 128, dtype=dtype)
                p = _plan(L, L.OP_BLOCK_FORWARD, dm, [0, T])
                big = dtype == L.BF16 and d % 256 == 0 and T >= 512
                assert p["ctx_fused_norm"] == int(big and p["ctx_splits"] == 1), (dtype, d, T, p)
                assert _plan(L, L.OP_BLOCK_LAYER, dm, [0, T])["ctx_fused_norm"] == 0
    dm = _dims(L, m=4, H=2560, d=1024, n_heads=8, dtype=L.BF16)
    assert _plan(L, L.OP_BLOCK_FORWARD, dm, [0, 16128])["ctx_fused_norm"] == 0    # 252 tiles: split
    p = _plan(L, L.OP_BLOCK_FORWARD, dm, [0, 16129])
    assert p["ctx_fused_norm"] == 1 and p["ctx_splits"] == 1                     # 256 tiles
    assert _plan(L, L.OP_CTX_FUSE, dm, [0, 131072])["ctx_fused_norm"] == 1
    assert _plan(L, L.OP_CTX_APPEND, dm, [0, 131072])["ctx_fused_norm"] == 1


def test_plan_splits_the_last_partial_round_of_eq2(L):
    """Fused Eq 2 tiles beyond whole rounds of 256 CUs: when they would fill at
    most half a round, their row tiles run as K splits (at most 256 / tiles,
    and no split narrower than 4 k-tiles); whole rounds and fuller last
    rounds keep one split."""
    dm = _dims(L, m=4, H=2560, d=1024, n_heads=8, dtype=L.BF16)
    for T in (16129, 20000, 131072, 131073, 184592, 200000, 245000):
        p = _plan(L, L.OP_BLOCK_FORWARD, dm, [0, T])
        tiles = -(-T // 256) * 4
        rest = tiles % 256
        want = (T - (tiles - rest) // 4 * 256) if 0 < rest <= 128 else 0
        assert p["ctx_fused_norm"] == 1 and p["ctx_tail_rows"] == want, (T, p)
    assert _plan(L, L.OP_BLOCK_FORWARD, dm, [0, 184592])["ctx_tail_rows"] == 4368
    # K = m*H too small for two splits of 4 k-tiles: no tail
    small = _dims(L, m=1, H=256, d=256, n_heads=2, dtype=L.BF16)
    assert _plan(L, L.OP_BLOCK_FORWARD, small, [0, 66000])["ctx_tail_rows"] == 0


def test_plan_reports_the_attention_path(L):
    """Long contexts take the streaming split-K kernel (more than 1024 64-key
    blocks over the heads), short ones the head-split kernel."""
    dm = _dims(L, m=2, H=128, d=256, n_heads=2, gamma=6)
    assert _plan(L, L.OP_BLOCK_FORWARD, dm, [0, 1000])["attn_streaming"] == 0
    p = _plan(L, L.OP_BLOCK_FORWARD, dm, [0, 30011, 30011, 41122])
    assert p["attn_streaming"] == 1 and p["attn_chunk"] > 64
    need = L.lib().dspark_workspace_size(L.OP_BLOCK_FORWARD, ctypes.byref(dm), 3, _cu([0, 30011, 30011, 41122]))
    assert p["workspace_bytes"] == need
