#!/usr/bin/env python3
"""Benchmark of the activation-sparse gated ReLU feedforward forward pass.

Default workload: one gated layer at the 1.5B-model shape (T = 8192 tokens,
d = 2048, F = 5632), bf16 inputs with fp32 accumulation, ~29 active
neurons per token, 1% outlier tokens with ~50% active neurons, TwELL tile
128 and capacity 8. Inputs are synthetic and seeded, resident in HBM
before the timed region. A step is one sparse forward: gate GEMM with the
ReLU + TwELL epilogue, overflow flags, fused sparse up/down projection and
the dense path for flagged rows.

Prints one JSON line: input tokens/ms, the same library's dense layer on
the same inputs, the roofline of the dominant kernel (timed with HIP
events on its own stream inside the timed region) and the CPU oracle timed
on a bounded sample on the host.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "input tokens/ms, sparse gated FFN fwd d=2048 ff=5632; % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix/vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def _dev(inp, name, torch, np):
    a = getattr(inp, name)
    if a is None:
        return None
    if inp.wl.dtype == "bf16":
        return torch.from_numpy(inp.bits(name).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _timed(fn, steps, warmup, torch, ffn=None):
    """Run warmup + timed steps; returns (ms per step, kernel profile)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    if ffn is not None:
        ffn.profile(True)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    ev = e0.elapsed_time(e1)
    prof = {}
    if ffn is not None:
        prof = ffn.profile_read()
        ffn.profile(False)
    return ev / steps, wall / steps, prof


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload (profiles/traffic_<workload>.json), for each kernel whose
    source file still hashes to what was profiled; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        rec = json.load(f)
    out = {}
    for kname, k in rec.get("kernels", {}).items():
        src = os.path.join(ROOT, "unstructured_sparse_feedforward_amd", "csrc", k["source"])
        try:
            h = hashlib.sha256(open(src, "rb").read()).hexdigest()
        except OSError:
            continue
        if h == k.get("source_sha256"):
            out[kname] = k["bytes_per_launch"]
    return out


def cpu_baseline(inp, sample, np):
    """The oracle's sparse forward (gate, TwELL pack, per-token up/down over
    active neurons, dense rows for flagged tokens) on the first `sample`
    tokens."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    w = inp.wl
    x = inp.x[:sample].astype(np.float64)
    wg = inp.w_gate.astype(np.float64).T
    wu = None if inp.w_up is None else inp.w_up.astype(np.float64).T
    wd = inp.w_down.astype(np.float64)
    t0 = time.perf_counter()
    oracle.sparse_ffn(x, wg, wu, wd, w.tile, w.twell_cap)
    ms = (time.perf_counter() - t0) * 1e3
    return {"value": sample / ms, "unit": "input tokens/ms", "cores": threads,
            "kind": "oracle",
            "sample": f"{sample} of {w.T} tokens, numpy float64 sparse forward "
                      f"(gate GEMM, TwELL pack, per-token up/down, dense flagged rows); "
                      f"{ms / 1e3:.1f} s; host os.cpu_count()={os.cpu_count()}"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gated",
                    choices=["gated", "nongated29", "nongated108", "nongated911", "small"])
    ap.add_argument("--cpu-sample", type=int, default=-1,
                    help="tokens of the oracle CPU baseline sample (-1 = all, 0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the timed work, run a plain elementwise copy of MIB MiB "
                         "(float32 negate into a second buffer) three times, so hardware "
                         "counters of the run can be scaled against known bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this layer is "
              "benchmarked on one MI355X; sharding is a design note, not a run mode.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from unstructured_sparse_feedforward_amd import SparseFFN
    from unstructured_sparse_feedforward_amd import workloads as wl

    W = {"gated": wl.GATED_1P5B, "small": wl.SMALL_F32, "nongated29": wl.NONGATED[29],
         "nongated108": wl.NONGATED[108], "nongated911": wl.NONGATED[911]}[args.workload]
    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    inp = wl.make_inputs(W, seed=args.seed)
    x, wg, wu, wd = (_dev(inp, k, torch, np) for k in ("x", "w_gate", "w_up", "w_down"))
    ffn = SparseFFN(W.d, W.F, gated=W.gated, twell_cap=W.twell_cap, tile=W.tile,
                    dtype=torch.bfloat16 if W.dtype == "bf16" else torch.float32)
    y = torch.empty((W.T, W.d), dtype=torch.float32, device="cuda")
    tw = ffn.new_twell(W.T)
    y_dense = torch.empty_like(y)

    sparse = lambda: ffn.forward(x, wg, wu, wd, mode="sparse", tw=tw, y=y)
    dense = lambda: ffn.forward(x, wg, wu, wd, mode="dense", y=y_dense)

    # timed region: K sparse steps, then K dense steps on the same inputs
    ms, wall_ms, _ = _timed(sparse, args.steps, args.warmup, torch, None)
    ms_d, wall_d, _ = _timed(dense, args.steps, args.warmup, torch, None)
    # the same steps again with every kernel bracketed by HIP events on the
    # launch stream, for the per-kernel durations
    ms_p, _, prof = _timed(sparse, args.steps, 0, torch, ffn)
    _, _, prof_d = _timed(dense, args.steps, 0, torch, ffn)

    # algorithmic work of the two main kernels
    torch.cuda.synchronize()
    cnt = tw["cnt"].cpu().numpy()
    flag = tw["row_flag"].cpu().numpy().astype(bool)
    n_flag = int(flag.sum())
    pairs = int(cnt[~flag].sum())
    esz = 2 if W.dtype == "bf16" else 4
    n_un = W.T - n_flag
    n_t = W.F // W.tile
    per_pair = (2 if W.gated else 1) * W.d * esz + 6          # weight rows + (val, idx)
    per_tok = W.d * esz + W.d * 4 + 4 * n_t + 1               # x, y, counts, flag
    gather_bytes = pairs * per_pair + n_un * per_tok
    gate_flops = 2.0 * W.T * W.d * W.F

    def avg(p, k):
        t, n = p.get(k, (0.0, 0))
        return t / n if n else float("nan")

    t_gate = avg(prof, "gate_gemm_twell")
    # the sparse up/down projection is two kernels (per-slice partial dot
    # products, then the down projection); its time is their sum
    t_gath = (avg(prof, "sparse_up") if W.gated else 0.0) + avg(prof, "sparse_down")
    peak_mm = PEAK_BF16_TFLOPS if W.dtype == "bf16" else PEAK_F32_TFLOPS
    roof_gate = {"bound": "mfma", "kernel": "gate_gemm_twell",
                 "achieved": gate_flops / (t_gate * 1e-3) / 1e12, "peak": peak_mm,
                 "unit": "TFLOP/s", "traffic": None, "avg_ms": t_gate}
    roof_gate["frac"] = roof_gate["achieved"] / peak_mm
    roof_gath = {"bound": "hbm", "kernel": "sparse_up + sparse_down",
                 "achieved": gather_bytes / (t_gath * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                 "unit": "GB/s", "traffic": None, "avg_ms": t_gath,
                 "algorithmic_bytes": gather_bytes, "active_pairs": pairs}
    roof_gath["frac"] = roof_gath["achieved"] / PEAK_HBM_GBS
    traffic = measured_traffic(W.name)
    if "gate_gemm_twell" in traffic:
        roof_gate["traffic"] = traffic["gate_gemm_twell"]
    if "sparse_up" in traffic and "sparse_down" in traffic:
        roof_gath["traffic"] = traffic["sparse_up"] + traffic["sparse_down"]
    dominant, other = (roof_gate, roof_gath) if t_gate >= t_gath else (roof_gath, roof_gate)

    out = {
        "metric": METRIC,
        "value": W.T / ms,
        "unit": "input tokens/ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.dtype,
        "data": "synthetic",
        "config": {"workload": W.name, "T": W.T, "d": W.d, "d_ff": W.F, "gated": W.gated,
                   "nnz_per_token": W.nnz, "twell_tile": W.tile, "twell_cap": W.twell_cap,
                   "outlier_frac": W.outlier_frac, "seed": args.seed},
        "roofline": dominant,
        "roofline_other": other,
        "dense_baseline": {"value": W.T / ms_d, "ms_per_step": ms_d,
                           "speedup_sparse_over_dense": ms_d / ms,
                           "kernels_avg_ms": {k: avg(prof_d, k) for k in prof_d}},
        "kernels_avg_ms": {k: avg(prof, k) for k in prof},
        "ms_per_step_wall": wall_ms,
        "ms_per_step_with_kernel_events": ms_p,
        "flagged_rows": n_flag,
    }
    if args.cpu_sample != 0:
        n = W.T if args.cpu_sample < 0 else min(args.cpu_sample, W.T)
        out["cpu_baseline"] = cpu_baseline(inp, n, np)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
