"""Throughput of the draft-block forward (Eq 2 + Eq 3) on one MI355X.

One step = one dspark_block_forward over one batch of synthetic context:
the Eq 2 fuse, the context K/V re-projection of every draft layer, and the
block side of every layer (projections, split-K attention + combine, SwiGLU
FFN, norms). Inputs are resident in HBM before the timed region.

Prints one JSON line: context tokens/s (value) and draft blocks/s, the
roofline of the dominant kernel (its average duration from HIP events taken
inside the timed region), and the CPU oracle timed on a bounded sample of the
same workload on the host cores.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-incremental]

The line also carries, under "incremental", the steady-state drafting regime
of the draft cache: one draft block over a cache of 8192 and of 131072
context rows (dspark_block_propose) and an 8-row append (dspark_ctx_append),
and under "markov" the greedy draft loop after the backbone
(dspark_markov_draft) for one and for 16 sequences.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import workloads as W  # noqa: E402

DEFAULT_WORKLOAD = "bf16-ragged16-L512..16384"
METRIC = "context tokens/s through Eq2+Eq3 and draft blocks/s; % MFMA / HBM peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def kernel_work(name, w, T, A):
    """Algorithmic work of ONE launch of a kernel kind: (amount, unit, bound).

    gemm_ctx_fuse  2*T*(m*H)*d flop          (Eq 2 projection)
    gemm_ctx_kv    2*T*d*(2*N*d) flop        (K and V of all N layers at once)
    attn_split_k   K_c + V_c of one layer (2*T*d*elt bytes) plus the queries
                   read and partials written (4 * A*gamma*d * 4 bytes)
    """
    esz = 2 if w.dtype == "bf16" else 4
    if name == "gemm_ctx_fuse":
        return 2.0 * T * w.m * w.H * w.d, "flop", "mfma"
    if name == "gemm_ctx_kv":
        return 2.0 * T * w.d * 2 * w.n_layers * w.d, "flop", "mfma"
    if name == "attn_split_k":
        return 2.0 * T * w.d * esz + 4.0 * A * w.gamma * w.d * 4, "byte", "hbm"
    return None


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gemm_ctx_fuse": ["block_draft_context_amd/csrc/gemm.hip", "block_draft_context_amd/csrc/common.h"],
    "gemm_ctx_kv": ["block_draft_context_amd/csrc/gemm.hip", "block_draft_context_amd/csrc/common.h",
                    "block_draft_context_amd/csrc/kv_layout.h"],
    "attn_split_k": ["block_draft_context_amd/csrc/attention.hip", "block_draft_context_amd/csrc/common.h",
                     "block_draft_context_amd/csrc/kv_layout.h"],
}


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, when
    it was taken on the current source of that kernel (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    e = rec.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return e.get("bytes_per_launch")


# rocprofv3 kernel names -> kernel kinds of the roofline (substring match)
PMC_KINDS = (("EpiKV", "gemm_ctx_kv"), ("EpiPartial", "gemm_ctx_fuse"), ("EpiNormBig", "gemm_ctx_fuse"),
             ("attn_partial_kernel", "attn_split_k"), ("attn_hsplit_kernel", "attn_split_k"))
CALIBRATION_KERNEL = "AUnaryFunctor"   # torch.mul(src, 1.0, out=dst) of --copy-calibration


def write_traffic(fetch_csv, write_csv, workload, copy_bytes):
    """HBM bytes per launch of the roofline kernels from two rocprofv3 --pmc
    runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each
    scaled so that the plain copy of --copy-calibration bytes reads and writes
    exactly copy_bytes; merged into profiles/hbm_traffic.json."""
    import csv
    import statistics

    def per_kind(path, counter):
        # median per kernel name, summed over the names of a kind: one call of
        # a kind may launch two kernels (the K/V product's 256x256 and 128x128
        # tiles)
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                kind = CALIBRATION_KERNEL if CALIBRATION_KERNEL in name else next(
                    (k for sub, k in PMC_KINDS if sub in name), None)
                if kind:
                    vals.setdefault(kind, {}).setdefault(name, []).append(float(r["Counter_Value"]) * 1024.0)
        return {k: sum(statistics.median(v) for v in names.values()) for k, names in vals.items()}

    fetch = per_kind(fetch_csv, "FETCH_SIZE")
    write = per_kind(write_csv, "WRITE_SIZE")
    f_scale = copy_bytes / fetch[CALIBRATION_KERNEL]
    w_scale = copy_bytes / write[CALIBRATION_KERNEL]
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    rec = {}
    if os.path.exists(path):
        with open(path) as f:
            rec = json.load(f)
    entry = rec.setdefault(workload, {})
    for kind in sorted(set(fetch) & set(write) - {CALIBRATION_KERNEL}):
        entry[kind] = {
            "fetch_bytes": round(fetch[kind] * f_scale),
            "write_bytes": round(write[kind] * w_scale),
            "bytes_per_launch": round(fetch[kind] * f_scale + write[kind] * w_scale),
            "source_hash": source_hash(KERNEL_SOURCES[kind]),
        }
    rec["calibration"] = {"copy_bytes": copy_bytes, "fetch_scale": round(f_scale, 4),
                          "write_scale": round(w_scale, 4)}
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps(rec[workload], indent=1))


def run_environment(B, torch):
    """What the line was measured on: device, software versions, host."""
    props = torch.cuda.get_device_properties(0)
    model, _ = host_cpu()
    return {"device": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "hip": torch.version.hip,
            "torch": torch.__version__, "library": B.version(), "host_cpu": model,
            "host_threads": len(os.sched_getaffinity(0))}


def host_cpu():
    """The host CPU model and the threads the oracle's BLAS uses."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    return model, int(threads)


def cpu_baseline(w, x, seconds, max_rows=32768):
    """The oracle (float32 mode) on a bounded sample of the workload: its
    first sequences up to about max_rows context rows (all of it when
    smaller), full forwards repeated until `seconds` of host time passed."""
    import oracle as O
    import numpy as np
    cu = [int(c) for c in x["cu"]]
    nb = 1
    while nb < w.A and cu[nb] < max_rows:
        nb += 1
    Ts = cu[nb]
    taps = [t[:Ts] for t in x["taps"]]
    cu_s = cu[:nb + 1]
    block_in = x["block_in"][:nb]
    model, threads = host_cpu()
    reps = 0
    O.block_forward(taps, x["w_c"], x["ctx_norm"], cu_s, block_in, x["block_pos"], x["layers"],
                    x["out_norm"], w.n_heads, w.eps, dtype=np.float32)   # untimed: page-in
    t0 = time.perf_counter()
    while True:
        O.block_forward(taps, x["w_c"], x["ctx_norm"], cu_s, block_in, x["block_pos"], x["layers"],
                        x["out_norm"], w.n_heads, w.eps, dtype=np.float32)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(reps * Ts / el, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "cpu_model": model,
            "draft_blocks_per_s": round(reps * nb / el, 3),
            "sample": (f"{reps} float32 numpy forwards of the first {nb} of {w.A} sequences of "
                       f"{w.name} (T={Ts} of {x['T']} context rows), {el:.1f} s")}


ROOF_KINDS = ("gemm_ctx_fuse", "gemm_ctx_kv", "attn_split_k")


def _time_calls(torch, call, stream, steps, warmup=3):
    """Per-call milliseconds (sorted) of `steps` back-to-back calls, from
    HIP events on the library's stream."""
    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


def bench_library_gemms(torch, w, steps):
    """Calibration, not the product: torch.matmul (hipBLASLt) on the two
    context products of the workload (the Eq 2 projection T x (m*H) -> d and
    the K/V of all layers T x d -> 2*N*d) on seeded bf16 operands, with plain
    bf16 output and none of the norms, row scales or attention layout, timed
    with HIP events on torch's stream. It marks what a tuned general GEMM
    reaches on the same shapes and part."""
    T = int(W.context_lengths(w).sum())
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(7)
    out = {"workload": w.name, "T": T}
    for name, (M, K, N) in (("gemm_ctx_fuse", (T, w.m * w.H, w.d)),
                            ("gemm_ctx_kv", (T, w.d, 2 * w.n_layers * w.d))):
        a = torch.randn(M, K, dtype=torch.bfloat16, device="cuda:0", generator=gen)
        b = torch.randn(N, K, dtype=torch.bfloat16, device="cuda:0", generator=gen)
        y = torch.empty(M, N, dtype=torch.bfloat16, device="cuda:0")
        bt = b.t()
        t = _time_calls(torch, lambda: torch.matmul(a, bt, out=y), torch.cuda.current_stream(), steps)
        ms = t[len(t) // 2]
        tflops = 2.0 * M * K * N / ms / 1e9
        out[name] = {"m_k_n": [M, K, N], "ms_median": round(ms, 4), "ms_min": round(t[0], 4),
                     "tflops": round(tflops, 1), "frac": round(tflops / PEAK_BF16_TFLOPS, 4)}
        del a, b, y, bt
    torch.cuda.empty_cache()
    return out


def bench_markov(B, torch, steps, vocab=131072, rank=256, gamma=5, d=1024, batches=(1, 16)):
    """The greedy draft loop after the backbone (dspark_markov_draft) for the
    5-position block of the d = 1024 drafter with a Markov rank of 256 (the
    module-dflash.ts defaults) over a 131072-entry vocabulary (the pages do
    not print one), for one and for 16 sequences. HBM-bound: each position
    streams w2 once for all sequences and moves the base and draft logits
    (algorithmic bytes per draft: gamma * (vocab * rank * 2 + 2 * A * vocab *
    4), that is w2, the base logits read and the draft logits written)."""
    out = {"vocab": vocab, "rank": rank, "gamma": gamma, "d": d}
    for A in batches:
        x = W.markov_inputs(90 + A, A=A, gamma=gamma, d=d, vocab=vocab, rank=rank)
        dev = "cuda:0"
        f = lambda a, t=torch.float32: torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=t)
        g = dict(block=f(x["block"]), U=f(x["base_logits"]), anchor=f(x["anchor"], torch.int32),
                 w1=f(x["w1"], torch.bfloat16), w2=f(x["w2"], torch.bfloat16), cw=f(x["conf_w"]),
                 cb=f(x["conf_b"]))
        dims = B.DsparkDims(m=1, H=64, d=d, n_heads=8, gamma=gamma, n_layers=1, ff=2 * d, dtype="bf16")
        toks = torch.empty((A, gamma), dtype=torch.int32, device=dev)
        conf = torch.empty((A, gamma), dtype=torch.float32, device=dev)
        logits = torch.empty((A, gamma, vocab), dtype=torch.float32, device=dev)
        call = lambda: B.markov_draft(dims, g["block"], g["U"], g["anchor"], g["w1"], g["w2"], g["cw"],
                                      g["cb"], tokens=toks, conf=conf, draft_logits=logits)
        t = _time_calls(torch, call, torch.cuda.current_stream(), steps)
        ms = t[len(t) // 2]
        amount = gamma * (vocab * rank * 2 + 2.0 * A * vocab * 4)
        out[f"A{A}"] = {"draft_ms_median": round(ms, 4), "draft_ms_min": round(t[0], 4),
                        "drafts_per_s": round(A * 1e3 / ms, 1),
                        "hbm": {"bound": "hbm", "achieved": round(amount / ms / 1e6, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(amount / ms / 1e6 / PEAK_HBM_GBS, 4)}}
        del g, logits
    torch.cuda.empty_cache()
    return out


def bench_incremental(B, torch, steps, lengths=(8192, 131072), new_rows=8):
    """The steady-state drafting regime of the incremental context: one
    sequence of the 5-layer d = 1024 drafter (the long-context workload's
    model), its draft cache filled to L context rows by dspark_ctx_append;
    then dspark_block_propose (one draft block over the cache) and an
    append of `new_rows` rows (the accepted tokens of a step) are timed at
    that length. Draft blocks/s = 1 / propose time."""
    from gpu_helpers import Uploaded, dims_of
    w = W.get_workload("bf16-L131072")
    x = W.make_inputs(w)
    u = Uploaded(w, x)
    del x
    dims = dims_of(B, w)
    cap = ((max(lengths) + new_rows + 63) // 64) * 64
    cache = B.DraftCache(dims, 1, cap)
    stream = torch.cuda.current_stream()
    out = {"workload": f"{w.name} drafter, one sequence", "new_rows_per_append": new_rows}
    done = 0
    for L in lengths:
        cache.append(u.taps[:, done:L], [L - done], u.w_c, u.ctx_norm, u.layers)
        done = L
        prop = B.prepared_propose(cache, u.block_in, u.block_pos, u.layers, u.out_norm)
        B.trace_begin(["attn_split_k"], capacity=(steps + 3) * 8)
        t = _time_calls(torch, prop, stream, steps)
        tr = B.trace_end().get("attn_split_k")
        app = B.prepared_append(cache, u.taps[:, 0:new_rows], [new_rows], u.w_c, u.ctx_norm, u.layers)
        ta = _time_calls(torch, app, stream, steps)
        rec = {"propose_ms_median": round(t[len(t) // 2], 4), "propose_ms_min": round(t[0], 4),
               "draft_blocks_per_s": round(1e3 / t[len(t) // 2], 1),
               "append_ms_median": round(ta[len(ta) // 2], 4),
               "draft_steps_per_s": round(1e3 / (t[len(t) // 2] + ta[len(ta) // 2]), 1)}
        if tr:
            amount = 2.0 * L * w.d * 2 + 4.0 * w.gamma * w.d * 4
            avg_s = tr[0] / tr[1] / 1e3
            rec["attention"] = {"bound": "hbm", "achieved": round(amount / avg_s / 1e9, 1),
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": round(amount / avg_s / 1e9 / PEAK_HBM_GBS, 4),
                                "avg_launch_us": round(avg_s * 1e6, 2)}
        out[f"L{L}"] = rec
    del cache, u
    torch.cuda.empty_cache()
    return out


def roofline_of(kind, w, T, A, total_ms, launches):
    """Roofline object of one kernel kind from its HIP-event totals."""
    amount, unit, bound = kernel_work(kind, w, T, A)
    avg_s = total_ms / launches / 1e3
    if unit == "flop":
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = amount / avg_s / 1e12
        runit = "TFLOP/s"
    else:
        peak = PEAK_HBM_GBS
        achieved = amount / avg_s / 1e9
        runit = "GB/s"
    return {"bound": bound, "kernel": kind, "achieved": round(achieved, 2), "peak": peak,
            "unit": runit, "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(kind, w.name),
            "avg_launch_us": round(avg_s * 1e6, 2), "launches_per_step": None,
            "work_per_launch": amount, "work_unit": unit}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(W.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-markov", action="store_true",
                    help="skip the greedy draft loop measurement (dspark_markov_draft)")
    ap.add_argument("--no-incremental", action="store_true",
                    help="skip the draft-cache measurement (propose / append at L = 8192, 131072)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--kernels", action="store_true", help="also print per-kernel times")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="first run a plain elementwise copy of BYTES bytes (3 launches), the "
                         "reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--library-gemms", action="store_true",
                    help="no forward: time torch.matmul (hipBLASLt) on the workload's two context "
                         "products with plain bf16 output, a calibration of what a tuned library "
                         "GEMM reaches on the same shapes, and print it as one JSON line")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no run: turn the counter_collection.csv files of two rocprofv3 --pmc "
                         "runs (FETCH_SIZE, WRITE_SIZE) of this script into profiles/hbm_traffic.json")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], args.workload,
                      args.copy_calibration or 268435456)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library runs on a single MI355X "
              "(no sharding or collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.library_gemms:
        print(json.dumps({"library_gemms": bench_library_gemms(torch, W.get_workload(args.workload),
                                                               max(args.steps, 5))}))
        return
    import block_draft_context_amd as B
    from gpu_helpers import Uploaded, dims_of

    if args.copy_calibration > 0:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst

    w = W.get_workload(args.workload)
    x = W.make_inputs(w)
    T, A = x["T"], w.A
    u = Uploaded(w, x)
    dims = dims_of(B, w)
    fwd = B.PreparedForward(dims, u.cu, u.taps, u.w_c, u.ctx_norm, u.block_in, u.block_pos,
                            u.layers, u.out_norm, cu_dev=u.cu_dev)
    names = B.kernel_names()

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()

    # untimed pass with every kind traced: per-kernel breakdown, dominant kernel
    B.trace_begin(names, capacity=4096)
    fwd()
    torch.cuda.synchronize()
    per_kind = B.trace_end()
    candidates = {k: v for k, v in per_kind.items() if k in ROOF_KINDS}
    dominant = max(candidates, key=lambda k: candidates[k][0])

    # timed region: K steps; HIP events around every launch of the three
    # roofline kernels (on the library's stream) and around each step
    roof_kinds = [k for k in ROOF_KINDS if k in per_kind]
    B.trace_begin(roof_kinds, capacity=args.steps * 32)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(fwd.stream)
        fwd()
        ev[i][1].record(fwd.stream)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    traced = B.trace_end()
    ms_per_step = el * 1e3 / args.steps
    step_ms = sorted(a.elapsed_time(b) for a, b in ev)

    rooflines = {}
    for k in roof_kinds:
        tot, n = traced[k]
        r = roofline_of(k, w, T, A, tot, n)
        r["launches_per_step"] = n // args.steps
        rooflines[k] = r

    res = {
        "metric": METRIC,
        "value": round(T / (ms_per_step / 1e3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_median": round(step_ms[len(step_ms) // 2], 4),
        "ms_per_step_min": round(step_ms[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) taps, N(0,0.02) weights)",
        "config": {"workload": w.name, "A": A, "T": T, "m": w.m, "H": w.H, "d": w.d,
                   "n_heads": w.n_heads, "gamma": w.gamma, "n_layers": w.n_layers, "ff": w.ff},
        "draft_blocks_per_s": round(A / (ms_per_step / 1e3), 2),
        "roofline": rooflines[dominant],
        "rooflines": rooflines,
    }
    # the context / block split of the step, from the event-traced pass
    ctx_kinds = ("gemm_ctx_fuse", "setup", "gemm_ctx_kv")
    t_ctx = sum(v[0] for k, v in per_kind.items() if k in ctx_kinds) / 1e3
    t_blk = sum(v[0] for k, v in per_kind.items() if k not in ctx_kinds) / 1e3
    res["context_side_tokens_per_s"] = round(T / t_ctx, 1) if t_ctx > 0 else None
    res["block_side_blocks_per_s"] = round(A / t_blk, 2) if t_blk > 0 else None
    proj = [k for k in ("gemm_ctx_fuse", "gemm_ctx_kv") if k in traced]
    if proj:
        flop = sum(kernel_work(k, w, T, A)[0] * traced[k][1] for k in proj)
        t_proj = sum(traced[k][0] for k in proj) / 1e3
        res["projections_frac_of_bf16_peak"] = round(flop / t_proj / 1e12 / PEAK_BF16_TFLOPS, 4)
    if args.kernels:
        res["kernels_us_per_step"] = {k: round(v[0] * 1e3, 2) for k, v in
                                      sorted(per_kind.items(), key=lambda kv: -kv[1][0])}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    if not args.no_incremental:
        del fwd, u, x
        torch.cuda.empty_cache()
        res["incremental"] = bench_incremental(B, torch, max(args.steps, 20))
    if not args.no_markov:
        res["markov"] = bench_markov(B, torch, max(args.steps, 20))
    res["env"] = run_environment(B, torch)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
