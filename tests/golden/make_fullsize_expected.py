"""Write the oracle's expected outputs for the full-size workloads.

Calls only ``oracle`` (float64) and the seeded generator ``workloads``. The
GPU parity tests regenerate the same inputs from the same seeds, check the
input fingerprints stored here, and compare the GPU outputs with:

  out      final normalised block rows [A, gamma, d]
  D1       block rows after the first draft layer [A, gamma, d]
  C_rows   sampled rows of the context memory H_ctx, at indices C_idx

Usage: python tests/golden/make_fullsize_expected.py [workload-name ...]
"""
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle as O  # noqa: E402
import workloads as W  # noqa: E402

N_SAMPLED_ROWS = 64


def fingerprint(x):
    h = hashlib.sha256()
    for t in x["taps"]:
        h.update(np.ascontiguousarray(t[:256]).tobytes())
        h.update(np.ascontiguousarray(t[-256:]).tobytes())
    h.update(x["w_c"].tobytes())
    h.update(x["layers"][-1]["w_down"].tobytes())
    h.update(x["block_in"].tobytes())
    h.update(x["block_pos"].tobytes())
    h.update(np.asarray(x["cu"], dtype=np.int64).tobytes())
    return h.hexdigest()


def expected_path(name):
    return os.path.join(HERE, "fullsize_" + name.replace("..", "-") + ".npz")


def make(name):
    w = W.get_workload(name)
    t0 = time.time()
    x = W.make_inputs(w)
    tr = {}
    out = O.block_forward(x["taps"], x["w_c"], x["ctx_norm"], x["cu"], x["block_in"],
                          x["block_pos"], x["layers"], x["out_norm"], w.n_heads, w.eps,
                          trace=tr)
    T = x["T"]
    idx = np.sort(np.random.default_rng(1234).choice(T, size=min(N_SAMPLED_ROWS, T), replace=False))
    np.savez_compressed(
        expected_path(name), out=out.astype(np.float32), D1=tr["D"][1].astype(np.float32),
        C_idx=idx.astype(np.int64), C_rows=tr["C"][idx].astype(np.float32),
        fingerprint=np.array(fingerprint(x)))
    print(f"{name}: T={T} written in {time.time() - t0:.1f}s", flush=True)


if __name__ == "__main__":
    names = sys.argv[1:] or [n for n, w in W.WORKLOADS.items() if w.dtype == "bf16"]
    for n in names:
        make(n)
