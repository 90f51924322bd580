"""Shared helpers of the GPU parity tests: upload seeded inputs, run the HIP
path through the C ABI, compare with the oracle."""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(got, ref) -> float:
    """Normwise max relative error ||y - r||_inf / ||r||_inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.max(np.abs(ref)), 1e-30))


def elem_rel_err(got, ref) -> float:
    """Elementwise relative error max |y - r| / max(|r|, 1e-3 ||r||_inf),
    reported for information next to the normwise bound."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    floor = 1e-3 * max(np.max(np.abs(ref)), 1e-30)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor)))


def dims_of(B, w):
    return B.DsparkDims(m=w.m, H=w.H, d=w.d, n_heads=w.n_heads, gamma=w.gamma,
                        n_layers=w.n_layers, ff=w.ff, eps=w.eps, dtype=w.dtype)


class Uploaded:
    """Device copies of one input set (storage dtype for the long tensors)."""

    def __init__(self, w, x, device="cuda:0"):
        import torch
        self.torch = torch
        dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.dt = dt
        f32 = torch.float32

        def up(a, t):
            return torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=t)

        T = x["T"]
        if "taps" in x:
            taps = torch.empty((w.m, T, w.H), dtype=dt, device=device)
            for j, t in enumerate(x["taps"]):
                taps[j].copy_(up(t, dt))
            self.taps = taps
        # the library takes every matrix [out, in] (y = x W^T); the oracle
        # keeps the [in, out] form of module-dflash.ts (y = x @ W)
        self.w_c = up(x["w_c"].T, dt)
        self.ctx_norm = up(x["ctx_norm"], f32)
        self.layers = [{k: up(v, f32) if k.endswith("norm") else up(v.T, dt) for k, v in lw.items()}
                       for lw in x["layers"]]
        self.block_in = up(x["block_in"], f32)
        self.block_pos = up(x["block_pos"], f32)
        self.out_norm = up(x["out_norm"], f32)
        self.cu = [int(c) for c in x["cu"]]
        self.cu_dev = torch.tensor(self.cu, dtype=torch.int32, device=device)


def oracle_forward(O, w, x, **kw):
    return O.block_forward(x["taps"], x["w_c"], x["ctx_norm"], x["cu"], x["block_in"],
                           x["block_pos"], x["layers"], x["out_norm"], w.n_heads, w.eps, **kw)
