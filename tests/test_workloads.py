"""The synthetic workloads against the sizes the pages print."""
import json
import os

import numpy as np

import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_default_drafter_shape_matches_page():
    cfg = _load("dflash_default_config.json")
    w = W.get_workload("bf16-L2048-d1024")
    assert w.m == len(cfg["tapLayers"])
    assert (w.d, w.n_heads, w.gamma, w.n_layers) == (cfg["dDraft"], cfg["nHeads"], cfg["gamma"], cfg["nLayers"])
    assert w.ff == cfg["ffMult"] * w.d
    for name in ("bf16-ragged16-L512..16384", "bf16-L131072"):
        v = W.get_workload(name)
        assert (v.m, v.d, v.n_heads, v.gamma, v.n_layers, v.ff) == (w.m, w.d, w.n_heads, w.gamma, w.n_layers, w.ff)


def test_five_tap_workload_matches_page():
    taps = _load("dspark_runtime_layers.json")["DSPARK_LAYERS"]
    assert W.get_workload("bf16-L8192-d2048-outliers").m == len(taps)


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 1.0 + 2**-9], dtype=np.float32)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa -> 1.0
    assert W.bf16_round(x).tolist() == [1.0, 1.0, 1.0 + 2**-6, -2.5, 1.0]


def test_inputs_are_deterministic_and_representable():
    w = W.small_workload(A=3, L_range=(0, 9), dtype="bf16", d=32, n_heads=2, H=16)
    a = W.make_inputs(w)
    b = W.make_inputs(w)
    for x, y in zip(a["taps"], b["taps"]):
        assert np.array_equal(x, y)
        assert np.array_equal(x, W.bf16_round(x))
    assert np.array_equal(a["layers"][0]["wq"], W.bf16_round(a["layers"][0]["wq"]))
    assert a["cu"][0] == 0 and np.all(np.diff(a["cu"]) >= 0)


def test_outlier_rows_and_ragged_lengths():
    w = W.get_workload("bf16-L8192-d2048-outliers")
    x = W.make_inputs(w, with_taps=False)
    assert x["T"] == 8192
    w4 = W.get_workload("bf16-ragged16-L512..16384")
    Ls = W.context_lengths(w4)
    assert Ls.shape == (16,) and Ls.min() >= 512 and Ls.max() <= 16384
