#!/usr/bin/env python3
"""Benchmark of the activation-sparse ReLU feedforward layer on one MI355X.

Default workload: one gated layer at the 1.5B-model shape (T = 8192 tokens,
d = 2048, F = 5632), bf16 inputs with fp32 accumulation, ~29 active
neurons per token, 1% outlier tokens with ~50% active neurons, TwELL tile
128 and capacity 8. Inputs are synthetic and seeded, resident in HBM
before the timed region. A step is one sparse forward: gate GEMM with the
ReLU + TwELL epilogue, row routing and ELL compaction, the dense path for
rows whose TwELL overflowed, and the sparse up/down projection.

Other workloads (--workload): the gated layer at 15 active neurons per
token (a stronger L1 stand-in, same shape); the non-gated layer at 29/108/911 active
neurons per token (F = 8192, T = 16384); the 18-layer gated stack
(T = 16384 per layer, active counts ramping 15 -> 120 -> 20, each layer on
its own seeded input); the training step (forward that saves the Hybrid
format, then the sparse backward: T = 8192, K = 64, 5% outliers); the small
fp32 layer.

Prints one JSON line: input tokens/ms, the same library's dense layer on
the same inputs (forward workloads), the roofline of the dominant kernel
(its launches bracketed by HIP events on their stream inside a timed pass)
and the CPU oracle timed on a bounded sample on the host.
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
METRIC_TRAIN = ("input tokens/ms, sparse gated FFN training step (fwd + bwd, Hybrid K=64) "
                "d=2048 ff=5632; % MFMA/HBM roofline")
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix/vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
# aggregate L2 read bandwidth, derived: 8 XCDs x 16 channels x 128 bytes
# per clock x 2.4 GHz (the L2 of a CDNA XCD: 4 MB in 16 channels of 128 B
# per clock). The sparse gathers are served from each XCD's L2 slice.
PEAK_L2_GBS = 8 * 16 * 128 * 2.4
SCRUB_BYTES = 2 << 30         # cold runs: bytes read between steps (> MALL + L2)

WORKLOADS = ("gated", "gated15", "nongated29", "nongated108", "nongated911", "stack18", "train",
             "small")


def _dev(inp, name, torch, np):
    a = getattr(inp, name)
    if a is None:
        return None
    if inp.wl.dtype == "bf16":
        return torch.from_numpy(inp.bits(name).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _timed(fn, steps, warmup, torch, ffns=(), per_step=None):
    """Warmup, then `steps` timed steps. Returns (event ms per step, wall ms
    per step, {kernel: (total ms, launches)} summed over `ffns` when they
    are given, whose launches are then bracketed by HIP events). With a
    list `per_step`, each step's own duration (an event before and after
    it) is appended to it."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    for f in ffns:
        f.profile(True)
    stream = torch.cuda.current_stream()
    ev_ = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    ev_[0].record(stream)
    for i in range(steps):
        fn()
        ev_[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    ev = ev_[0].elapsed_time(ev_[-1])
    if per_step is not None:
        per_step.extend(ev_[i].elapsed_time(ev_[i + 1]) for i in range(steps))
    prof = {}
    for f in ffns:
        for k, (ms, n) in f.profile_read().items():
            a, b = prof.get(k, (0.0, 0))
            prof[k] = (a + ms, b + n)
        f.profile(False)
    return ev / steps, wall / steps, prof


def _timed_cold(fn, steps, torch, scrub):
    """`steps` steps, each after a read of the whole scrub buffer (larger
    than the Infinity Cache and the L2s together), so every step starts
    with its inputs and weights in HBM only. Returns each step's duration
    (events right before and after it)."""
    out = []
    stream = torch.cuda.current_stream()
    for _ in range(steps):
        torch.sum(scrub)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return out


def pct(v):
    """Median, p10 and p90 of per-step milliseconds."""
    import numpy as np
    a = np.asarray(v, dtype=np.float64)
    return {"p10": float(np.percentile(a, 10)), "median": float(np.median(a)),
            "p90": float(np.percentile(a, 90)), "n": int(a.size)}


def measured_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload (profiles/traffic_<workload>.json), for each kernel whose
    source file still hashes to what was profiled."""
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


def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return os.cpu_count()


# host time the CPU baseline spends on its sample (the oracle runs over the
# sample again until this much has passed)
CPU_MIN_MS = 10000.0


def repeat_ms(fn, min_ms):
    """Run fn once and then again until min_ms of host time has passed (at
    most 64 runs): (total ms, runs)."""
    total, runs = 0.0, 0
    while runs == 0 or (total < min_ms and runs < 64):
        t0 = time.perf_counter()
        fn()
        total += (time.perf_counter() - t0) * 1e3
        runs += 1
    return total, runs


def oracle_forward_ms(inp, n, np, min_ms=0.0):
    """Host ms of the oracle's sparse forward (gate GEMM, TwELL pack,
    per-token up/down over the active neurons, dense rows for flagged
    tokens) on the first n tokens of one layer, repeated until min_ms:
    (total ms, runs)."""
    import oracle
    w = inp.wl
    x = inp.x[:n].astype(np.float64)
    wg = inp.w_gate.astype(np.float64).T
    wu = None if inp.w_up is None else inp.w_up.astype(np.float64).T
    wd = inp.w_down.astype(np.float64)
    return repeat_ms(lambda: oracle.sparse_ffn(x, wg, wu, wd, w.tile, w.twell_cap), min_ms)


def _host():
    """The host the oracle ran on: CPU model and the BLAS numpy calls."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = [{"api": i.get("internal_api"), "threads": i.get("num_threads"),
                 "arch": i.get("architecture")} for i in threadpool_info()
                if i.get("user_api") == "blas"]
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "blas": blas}


def cpu_record(tokens, ms, sample):
    return {"value": tokens / ms, "unit": "input tokens/ms", "cores": _threads(),
            "kind": "oracle",
            "sample": f"{sample}; {ms / 1e3:.1f} s; host os.cpu_count()={os.cpu_count()}",
            "host": _host()}


def gather_work(W, cnt, flag, np, ssz=4):
    """Algorithmic bytes of the sparse up/down projection of one layer:
    per active pair of an unflagged row the weight rows it reads and its
    (value, index) (ssz: bytes of a stored value); per unflagged row its x
    row, y row, tile counts, flag."""
    n_flag = int(flag.sum())
    pairs = int(cnt[~flag].sum())
    esz = 2 if W.dtype == "bf16" else 4
    n_t = W.F // W.tile
    per_pair = (2 if W.gated else 1) * W.d * esz + ssz + 2
    per_tok = W.d * esz + W.d * 4 + 4 * n_t + 1
    return pairs * per_pair + (W.T - n_flag) * per_tok, pairs, n_flag


def roof(kind, name, work, prof, keys, peak, traffic=None):
    """Roofline record of one kernel (or of consecutive kernels that
    together make one step of the path) from its per-launch average:
    `work` is the algorithmic FLOP ("mfma") or bytes ("hbm") over all the
    launches the profile counted."""
    ms = sum(prof.get(k, (0.0, 0))[0] for k in keys)
    n = max([prof.get(k, (0.0, 0))[1] for k in keys] + [0])
    if n == 0 or ms <= 0:
        return None
    per_launch_ms = ms / n
    w = work / n
    ach = w / (per_launch_ms * 1e-3) / (1e12 if kind == "mfma" else 1e9)
    r = {"bound": kind, "kernel": name, "achieved": ach, "peak": peak,
         "unit": "TFLOP/s" if kind == "mfma" else "GB/s", "frac": ach / peak,
         "traffic": traffic, "avg_ms": per_launch_ms, "launches": n}
    r["algorithmic_flop" if kind == "mfma" else "algorithmic_bytes"] = w
    return r


def _socket_power_w():
    """One reading of the GPU's socket power (amd-smi), or None."""
    import re
    import subprocess
    try:
        out = subprocess.run(["amd-smi", "metric", "--power", "-g", "0"], capture_output=True,
                             text=True, timeout=10).stdout
    except Exception:
        return None
    m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", out)
    return float(m.group(1)) if m else None


def measure_energy(fn, tokens, torch, seconds=3.0):
    """Average socket power while fn runs back to back for about `seconds`
    (amd-smi sampled from a host thread) and the energy per input token."""
    import threading
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            p = _socket_power_w()
            if p is not None:
                samples.append(p)
            stop.wait(0.1)

    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    th = threading.Thread(target=sampler)
    th.start()
    steps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        steps += 10
        torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stop.set()
    th.join()
    if not samples:
        return None
    p = sum(samples) / len(samples)
    return {"power_W": p, "samples": len(samples), "steps": steps,
            "uJ_per_token": p * elapsed / (steps * tokens) * 1e6}


def probe_rates(torch):
    """Device rates from libsffn_probe.so (sffn_probe_rates), in GB/s per CU,
    or None when the probe library is not built."""
    import ctypes
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "unstructured_sparse_feedforward_amd", "libsffn_probe.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.sffn_probe_rates.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_double), ctypes.c_int]
    lib.sffn_probe_rates.restype = ctypes.c_int
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    out = (ctypes.c_double * 5)()
    st = lib.sffn_probe_rates(n_cu, out, 5)
    torch.cuda.synchronize()
    if st != 0:
        raise RuntimeError(f"sffn_probe_rates failed with HIP error {st}")
    keys = ("lds_reads", "lds_copies", "lds_reads_and_copies", "loads_row_pieces",
            "loads_mfma_layout")
    return {"unit": "GB/s per CU", "num_cu": n_cu,
            **{k: out[i] / 1e9 for i, k in enumerate(keys)},
            "note": "lds_*: 16-byte ds_read_b128 fragment reads and 16-byte direct-to-LDS "
                    "copies (L2-resident source), alone and issued together (both kinds "
                    "summed); loads_*: 16-byte L2-to-register loads, four lanes per 64-byte "
                    "row piece vs the 32x32 MFMA operand layout"}


def gate_lds_bytes(T, d, F):
    """LDS bytes one launch of the bf16 gate GEMM + TwELL kernel moves: 256 x
    256 tiles, each ring stage (32 k) copied into LDS once (256 + 256 rows x
    64 B), and each of the 4 waves reading 4 A and 4 B 16-byte fragments
    (1 KB per wave each) per 16 k: (copy bytes, read bytes). The epilogue's
    staging reads (16 KB per wave and 32-row block) are not counted."""
    tiles = -(-T // 256) * -(-F // 256)
    copies = tiles * (256 + 256) * d * 2
    reads = tiles * 4 * (d // 16) * 8 * 1024
    return copies, reads


def per_step(prof, steps):
    return {k: ms / steps for k, (ms, n) in prof.items()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gated", choices=WORKLOADS)
    ap.add_argument("--cpu-sample", type=int, default=-1,
                    help="tokens of the oracle CPU baseline sample (-1 = the workload's "
                         "default, 0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--energy", action=argparse.BooleanOptionalAction, default=True,
                    help="run the sparse and dense forwards for ~3 s each while sampling the "
                         "socket power with amd-smi, and report energy per token (default on)")
    ap.add_argument("--store", default="f32", choices=("f32", "bf16"),
                    help="dtype of the stored activations (TwELL values, Hybrid a and u)")
    ap.add_argument("--updown", default="sliced", choices=("sliced", "fused"),
                    help="inference up/down: three XCD-sliced launches (default) or the one "
                         "fused kernel without slices")
    ap.add_argument("--graph", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the sparse step captured once as a HIP graph and "
                         "replayed (forward workloads)")
    ap.add_argument("--cold-steps", type=int, default=20,
                    help="cold-cache steps of each mode (a 2 GiB read before each; 0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="before the timed work, run a plain elementwise copy of MIB MiB "
                         "(float32 negate into a second buffer) three times, so hardware "
                         "counters of the run can be scaled against known bytes")
    args = ap.parse_args()
    if args.store == "bf16" and args.workload == "small":
        print("--store bf16 serves bf16 layers; the small workload is fp32", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this layer is "
              "benchmarked on one MI355X; sharding is a design note, not a run mode.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from unstructured_sparse_feedforward_amd import SparseFFN
    from unstructured_sparse_feedforward_amd import workloads as wl

    torch.cuda.set_device(0)
    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    if args.workload == "train":
        out = bench_train(args, np, torch, SparseFFN, wl)
    elif args.workload == "stack18":
        out = bench_stack(args, np, torch, SparseFFN, wl)
    else:
        out = bench_forward(args, np, torch, SparseFFN, wl)
    print(json.dumps(out), flush=True)
    return 0


def bench_forward(args, np, torch, SparseFFN, wl):
    Ws = [{"gated": wl.GATED_1P5B, "gated15": wl.GATED_1P5B_NNZ15,
           "small": wl.SMALL_F32, "nongated29": wl.NONGATED[29],
           "nongated108": wl.NONGATED[108],
           "nongated911": wl.NONGATED[911]}[args.workload]]
    W0 = Ws[0]
    if args.cpu_sample < 0:
        n_cpu = 2048 if W0.F == 8192 else W0.T
    else:
        n_cpu = min(args.cpu_sample, W0.T)
    layers, cpu_ms, cpu_runs = [], 0.0, 0
    for i, W in enumerate(Ws):
        inp = wl.make_inputs(W, seed=args.seed, layer=i)
        # the oracle's host time on this layer's first n_cpu tokens
        if n_cpu > 0:
            ms_, cpu_runs = oracle_forward_ms(inp, n_cpu, np, CPU_MIN_MS / len(Ws))
            cpu_ms += ms_
        ffn = SparseFFN(W.d, W.F, gated=W.gated, twell_cap=W.twell_cap, tile=W.tile,
                        ell_cap=W.ell_cap, dense_rows=W.dense_rows,
                        dtype=torch.bfloat16 if W.dtype == "bf16" else torch.float32,
                        store_dtype=_store(args, torch), fused_updown=args.updown == "fused")
        y = torch.empty((W.T, W.d), dtype=torch.float32, device="cuda")
        layers.append(dict(W=W, ffn=ffn, tw=ffn.new_twell(W.T), y=y, yd=torch.empty_like(y),
                           args=[_dev(inp, k, torch, np)
                                 for k in ("x", "w_gate", "w_up", "w_down")]))
        del inp

    def sparse():
        for L in layers:
            L["ffn"].forward(*L["args"], mode="sparse", tw=L["tw"], y=L["y"], check=False)

    def dense():
        for L in layers:
            L["ffn"].forward(*L["args"], mode="dense", y=L["yd"], check=False)

    # one checked pass first: every routed row fits the dense path's capacity
    for L in layers:
        L["ffn"].forward(*L["args"], mode="sparse", tw=L["tw"], y=L["y"])
        if L["ffn"].dense_rows != L["W"].dense_rows:
            raise RuntimeError(f"{L['W'].name}: more rows took the dense path than "
                               f"dense_rows = {L['W'].dense_rows}")

    ffns = [L["ffn"] for L in layers]
    # timed region: K sparse steps, then K dense steps on the same inputs
    # (warm: inputs and weights may stay in the caches between steps)
    sp_steps, de_steps = [], []
    ms, wall_ms, _ = _timed(sparse, args.steps, args.warmup, torch, per_step=sp_steps)
    ms_d, _, _ = _timed(dense, args.steps, args.warmup, torch, per_step=de_steps)
    # the same steps again with every kernel bracketed by HIP events on the
    # launch stream, for the per-kernel durations
    ms_p, _, prof = _timed(sparse, args.steps, 0, torch, ffns)
    _, _, prof_d = _timed(dense, args.steps, 0, torch, ffns)
    torch.cuda.synchronize()
    for f in ffns:
        f.check()
    # cold: every step after a 2 GiB read that evicts the caches
    cold = None
    if args.cold_steps > 0:
        scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device="cuda")
        sp_cold = _timed_cold(sparse, args.cold_steps, torch, scrub)
        de_cold = _timed_cold(dense, args.cold_steps, torch, scrub)
        del scrub
        cold = {"method": f"each step after torch.sum over a {SCRUB_BYTES >> 30} GiB buffer "
                          "(evicts the 256 MB Infinity Cache and the L2s); events around the "
                          "step alone",
                "sparse_ms": pct(sp_cold), "dense_ms": pct(de_cold),
                "value": T_of(layers) / pct(sp_cold)["median"],
                "dense_value": T_of(layers) / pct(de_cold)["median"],
                "speedup_sparse_over_dense": pct(de_cold)["median"] / pct(sp_cold)["median"]}

    # the same sparse step captured once as a HIP graph (torch.cuda.CUDAGraph
    # over the library's launches on the capturing stream) and replayed:
    # the same kernels without the host's per-launch overhead; every
    # replayed y is compared bit for bit with the eager step's
    graph = None
    if args.graph:
        ref = [L["y"].clone() for L in layers]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            sparse()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sparse()
        g_steps = []
        ms_g, _, _ = _timed(g.replay, args.steps, args.warmup, torch, per_step=g_steps)
        torch.cuda.synchronize()
        same = all(torch.equal(L["y"].view(torch.int32), r.view(torch.int32))
                   for L, r in zip(layers, ref))
        del g
        graph = {"ms_per_step": ms_g, "value": T_of(layers) / ms_g, "step_ms": pct(g_steps),
                 "same_y_as_eager": bool(same),
                 "method": "torch.cuda.CUDAGraph capture of one sparse step, replayed; "
                           "events around the timed replays"}

    gbytes, pairs, n_flag = 0.0, 0, 0
    for L in layers:
        b, p, nf = gather_work(L["W"], L["tw"]["cnt"].cpu().numpy(),
                               L["tw"]["row_flag"].cpu().numpy().astype(bool), np,
                               ssz=2 if args.store == "bf16" else 4)
        gbytes += b
        pairs += p
        n_flag += nf
    flops = sum(2.0 * W.T * W.d * W.F for W in Ws)
    # the dense layer: gate, up and down products (non-gated: two)
    dense_flops = sum(2.0 * W.T * W.d * W.F * (3 if W.gated else 2) for W in Ws)
    peak_mm = PEAK_BF16_TFLOPS if W0.dtype == "bf16" else PEAK_F32_TFLOPS
    traffic = measured_traffic(W0.name)
    r_gate = roof("mfma", "gate_gemm_twell", flops * args.steps, prof, ["gate_gemm_twell"],
                  peak_mm, traffic.get("gate_gemm_twell"))
    rates = probe_rates(torch)
    torch_ffn = None
    if W0.dtype == "bf16":
        # the gate GEMM's operand copies into LDS and its fragment reads,
        # each against the rate probed on this device
        cb, rb = gate_lds_bytes(W0.T, W0.d, W0.F)
        per_s = (r_gate["avg_ms"] * 1e-3) * 1e9 * (rates["num_cu"] if rates else 256)
        r_gate["lds"] = {
            "copy_bytes_per_launch": cb, "read_bytes_per_launch": rb, "unit": "GB/s per CU",
            "copies_per_cu": cb / per_s, "reads_per_cu": rb / per_s,
            "copy_frac": cb / per_s / rates["lds_copies"] if rates else None,
            "read_frac": rb / per_s / rates["lds_reads"] if rates else None,
            "note": "direct-to-LDS operand copies and 16-byte fragment reads per launch, "
                    "against the probed rates of each (device_rates)"}
        # context, not part of the path: the vendor bf16 GEMM (torch linear,
        # hipBLASLt) on the gate's shape, plain output, no epilogue, and
        # torch's own bf16 dense layer (two or three linear calls with the
        # ReLU and product between them)
        x0, wg0, wu0, wd0 = layers[0]["args"]
        vms = _torch_ms(lambda: torch.nn.functional.linear(x0, wg0), args.steps, torch)
        vflop = 2.0 * W0.T * W0.d * W0.F
        r_gate["vendor_gemm_same_shape"] = {
            "kernel": "torch.nn.functional.linear bf16 (hipBLASLt), bf16 output, no epilogue",
            "avg_ms": vms, "achieved": vflop / (vms * 1e-3) / 1e12,
            "frac": vflop / (vms * 1e-3) / 1e12 / peak_mm}
        wdT = wd0.t().contiguous()
        F_ = torch.nn.functional

        def torch_dense():
            h = F_.relu(F_.linear(x0, wg0))
            if wu0 is not None:
                h = h * F_.linear(x0, wu0)
            return F_.linear(h, wdT)

        tms = _torch_ms(torch_dense, args.steps, torch)
        del wdT
        torch_ffn = {"kernel": "torch bf16 dense layer: linear, relu, linear, mul, linear "
                               "(hipBLASLt GEMMs, bf16 output)",
                     "ms_per_step": tms, "value": W0.T / tms,
                     "frac_of_bf16_peak": dense_flops / (tms * 1e-3) / 1e12 / peak_mm}
    # the sparse up/down projection is three kernels (per-slice partial dot
    # products, their sums h = a * u, the down projection); a launch of it
    # is one of each
    keys = ["sparse_up", "sparse_hsum", "sparse_down"] if W0.gated else ["sparse_down"]
    if args.updown == "fused":
        keys = ["fused_updown"]
    tr = sum(traffic[k] for k in keys) if all(k in traffic for k in keys) else None
    r_gath = roof("hbm", " + ".join(keys), gbytes * args.steps, prof, keys, PEAK_HBM_GBS, tr)
    r_gath["active_pairs_per_step"] = pairs
    # the algorithmic bytes are what the path gathers; most of them are
    # served by the XCDs' L2s (each XCD gathers from one 2.9 MB slice of the
    # weights at a time), so the frac above is an effective rate. Against
    # what bounds it: the aggregate L2 bandwidth, and the HBM side measured
    # by the committed counters
    r_gath["l2_relative"] = {"peak": PEAK_L2_GBS, "unit": "GB/s",
                             "frac": r_gath["achieved"] / PEAK_L2_GBS,
                             "peak_note": "derived: 8 XCDs x 16 L2 channels x 128 B/clk x "
                                          "2.4 GHz"}
    r_gath["hbm_side"] = None if tr is None else {
        "bytes_per_launch": tr, "achieved": tr / (r_gath["avg_ms"] * 1e-3) / 1e9,
        "frac": tr / (r_gath["avg_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, "unit": "GB/s",
        "source": "rocprofv3 FETCH_SIZE + WRITE_SIZE of the three kernels (profiles/)"}
    dominant, other = ((r_gate, r_gath) if r_gate["avg_ms"] >= r_gath["avg_ms"]
                       else (r_gath, r_gate))
    T = W0.T
    cfg = {"workload": W0.name, "T": T, "d": W0.d, "d_ff": W0.F, "gated": W0.gated,
           "nnz_per_token": W0.nnz, "twell_tile": W0.tile, "twell_cap": W0.twell_cap,
           "ell_cap": W0.ell_cap, "dense_rows": W0.dense_rows, "store_dtype": args.store,
           "updown": args.updown,
           "outlier_frac": W0.outlier_frac, "seed": args.seed}
    out = {
        "metric": METRIC,
        "value": T / ms,
        "unit": "input tokens/ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W0.dtype,
        "data": "synthetic",
        "config": cfg,
        "roofline": dominant,
        "roofline_other": other,
        "step_ms": pct(sp_steps),
        "dense_baseline": {"value": T / ms_d, "ms_per_step": ms_d, "step_ms": pct(de_steps),
                           "speedup_sparse_over_dense": ms_d / ms,
                           "frac_of_mfma_peak": dense_flops / (ms_d * 1e-3) / 1e12 / peak_mm,
                           "kernels_ms_per_step": per_step(prof_d, args.steps)},
        "cold": cold,
        "graph": graph,
        "device_rates": rates,
        "torch_dense_layer": torch_ffn,
        "kernels_ms_per_step": per_step(prof, args.steps),
        "ms_per_step_wall": wall_ms,
        "ms_per_step_with_kernel_events": ms_p,
        "flagged_rows_per_step": n_flag,
        "device_bytes": forward_bytes(layers),
    }
    if args.energy:
        idle = _socket_power_w()
        e_sp = measure_energy(sparse, T, torch)
        e_de = measure_energy(dense, T, torch)
        out["energy"] = None if e_sp is None or e_de is None else {
            "idle_W": idle, "sparse": e_sp, "dense": e_de,
            "sparse_over_dense": e_sp["uJ_per_token"] / e_de["uJ_per_token"],
            "method": "amd-smi socket power sampled every ~0.1-0.3 s from a host thread "
                      "while the forward runs back to back for ~3 s"}
    if n_cpu > 0:
        what = f"first {n_cpu} of {T} tokens, {cpu_runs} run(s)"
        out["cpu_baseline"] = cpu_record(
            n_cpu * cpu_runs, cpu_ms,
            f"{what}: numpy float64 sparse forward (gate GEMM, TwELL pack, per-token "
            f"up/down over active neurons, dense flagged rows)")
    return out


def _store(args, torch):
    return torch.bfloat16 if args.store == "bf16" else torch.float32


def T_of(layers):
    return layers[0]["W"].T


def _torch_ms(fn, steps, torch):
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def forward_bytes(layers):
    """Device bytes one layer's forward holds beyond its inputs and y: the
    library's workspace (and the TwELL the bench passes in) for the sparse
    forward, the workspace (the bf16 hidden tensor) for the dense one."""
    from unstructured_sparse_feedforward_amd import binding as B
    L = layers[0]
    f, W = L["ffn"], L["W"]
    tw = sum(t.numel() * t.element_size() for t in L["tw"].values())
    return {"sparse_workspace": f.workspace_bytes(W.T, B.SFFN_OP_FORWARD_SPARSE),
            "sparse_twell": tw,
            "dense_workspace": f.workspace_bytes(W.T, B.SFFN_OP_FORWARD_DENSE)}


def bench_stack(args, np, torch, SparseFFN, wl):
    """The 18-layer stack chained with residual connections and RMS
    normalisation: every layer sparse, every layer dense, and each layer in
    the mode the library picks from its own TwELL (sffn_choose_mode); each
    layer's two modes are also timed alone on its chained input, to check
    the library's choices."""
    from unstructured_sparse_feedforward_amd.stack import FFNStack
    Ws = [wl.stack_layer(i) for i in range(len(wl.STACK_RAMP))]
    T = Ws[0].T
    n_cpu = 256 if args.cpu_sample < 0 else min(args.cpu_sample, T)
    weights, cpu_ms, cpu_tok = [], 0.0, 0
    for i, W in enumerate(Ws):
        inp = wl.make_inputs(W, seed=args.seed, layer=i)
        if i == 0:
            x0, outlier = inp.x, inp.outlier
        if n_cpu > 0:
            ms_, runs_ = oracle_forward_ms(inp, n_cpu, np, CPU_MIN_MS / len(Ws))
            cpu_ms += ms_
            cpu_tok += n_cpu * runs_
        weights.append(tuple(_dev(inp, k, torch, np) for k in ("w_gate", "w_up", "w_down")))
        del inp
        print(f"layer {i} on the device", file=sys.stderr, flush=True)
    stack = FFNStack(weights, Ws, T, store_dtype=_store(args, torch))
    keep = torch.from_numpy((~outlier).astype(np.float32)).to(torch.bfloat16).cuda()
    h0 = torch.from_numpy(x0).cuda()
    info = stack.choose_modes(h0, keep)
    chosen = list(stack.modes)
    tw_counts = [(t["cnt"].cpu().numpy(), t["row_flag"].cpu().numpy().astype(bool))
                 for t in stack.tw]

    def run():
        stack.forward(h0, keep)

    res = {}
    for name, modes in (("sparse", ["sparse"] * len(Ws)), ("dense", ["dense"] * len(Ws)),
                        ("chosen", chosen)):
        stack.modes = modes
        steps_ms = []
        ms, _, _ = _timed(run, args.steps, args.warmup, torch, per_step=steps_ms)
        res[name] = {"ms_per_step": ms, "value": T / ms, "step_ms": pct(steps_ms)}
    stack.modes = ["sparse"] * len(Ws)
    ms_p, _, prof = _timed(run, args.steps, 0, torch, stack.ffns)
    stack.check()
    # each layer alone on its chained input, in both modes
    rec = []
    stack.forward(h0, keep, record=rec)
    alone = []
    for l, (f, w) in enumerate(zip(stack.ffns, stack.weights)):
        x = rec[l][0]
        y = torch.empty((T, Ws[l].d), dtype=torch.float32, device="cuda")
        t_sp = _torch_ms(lambda: f.forward(x, *w, mode="sparse", tw=stack.tw[l], y=y,
                                           check=False), 10, torch)
        t_de = _torch_ms(lambda: f.forward(x, *w, mode="dense", y=y, check=False), 10, torch)
        alone.append((t_sp, t_de))
    del rec
    stack.check()
    gbytes, pairs, n_flag = 0.0, 0, 0
    for W, (cnt, flag) in zip(Ws, tw_counts):
        b, p, nf = gather_work(W, cnt, flag, np, ssz=2 if args.store == "bf16" else 4)
        gbytes += b
        pairs += p
        n_flag += nf
    flops = sum(2.0 * W.T * W.d * W.F for W in Ws)
    r_gate = roof("mfma", "gate_gemm_twell", flops * args.steps, prof, ["gate_gemm_twell"],
                  PEAK_BF16_TFLOPS)
    keys = ["sparse_up", "sparse_hsum", "sparse_down"]
    r_gath = roof("hbm", " + ".join(keys), gbytes * args.steps, prof, keys, PEAK_HBM_GBS)
    r_gath["l2_relative"] = {"peak": PEAK_L2_GBS, "unit": "GB/s",
                             "frac": r_gath["achieved"] / PEAK_L2_GBS}
    W0 = Ws[0]
    ms = res["sparse"]["ms_per_step"]
    layers = [{"layer": l, "target_active": W.nnz, "mean_active": m, "crossover": c,
               "chosen": mode, "alone_ms_sparse": a[0], "alone_ms_dense": a[1],
               "faster_alone": "sparse" if a[0] <= a[1] else "dense"}
              for l, (W, (mode, m, c), a) in enumerate(zip(Ws, info, alone))]
    out = {
        "metric": "input tokens/ms through 18 sparse gated FFN layers (fwd) d=2048 ff=5632; "
                  "% MFMA/HBM roofline",
        "value": T / ms,
        "unit": "input tokens/ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W0.dtype,
        "data": "synthetic",
        "config": {"workload": wl.STACK_LAYER.name, "T": T, "d": W0.d, "d_ff": W0.F,
                   "layers": len(Ws), "nnz_per_token": list(wl.STACK_RAMP),
                   "twell_cap": W0.twell_cap, "ell_cap": W0.ell_cap,
                   "dense_rows": W0.dense_rows, "store_dtype": args.store,
                   "outlier_frac": W0.outlier_frac, "front_positions": W0.front_positions,
                   "front_prob": W0.front_prob, "seq_len": W0.seq_len,
                   "chaining": "h += FFN(RMSNorm(h)) per layer (column 0: bias input)",
                   "seed": args.seed},
        "roofline": r_gate,
        "roofline_other": r_gath,
        "step_ms": res["sparse"]["step_ms"],
        "dense_baseline": dict(res["dense"], speedup_sparse_over_dense=
                               res["dense"]["ms_per_step"] / ms),
        "dispatch": dict(res["chosen"], modes=chosen,
                         speedup_over_dense=res["dense"]["ms_per_step"] /
                         res["chosen"]["ms_per_step"],
                         choices_matching_alone_timing=sum(
                             L["chosen"] == L["faster_alone"] for L in layers),
                         rule="sffn_choose_mode: dense iff the layer's mean active neurons "
                              "per token (non-overflowing rows) exceeds the cost-model "
                              "crossover"),
        "layers": layers,
        "kernels_ms_per_step": per_step(prof, args.steps),
        "ms_per_step_with_kernel_events": ms_p,
        "flagged_rows_per_step": n_flag,
        "active_pairs_per_step": pairs,
    }
    if n_cpu > 0:
        out["cpu_baseline"] = cpu_record(
            cpu_tok / len(Ws), cpu_ms,
            f"first {n_cpu} tokens of each of the {len(Ws)} layers, each layer's oracle run "
            f"until {CPU_MIN_MS / len(Ws) / 1e3:.2f} s (on the layer's own seeded input, whose "
            f"values do not change the oracle's cost): numpy float64 sparse forward (gate "
            f"GEMM, TwELL pack, per-token up/down over active neurons, dense flagged rows); "
            f"tokens/ms through all {len(Ws)} layers")
    return out


def dense_train(ffn, a, dy, grads, args, torch):
    """The same library's dense bf16 training step of the layer
    (sffn_forward_train_dense + sffn_backward_dense): time per step, the
    bytes of its saved activations and the device memory one step adds to
    the inputs and weights (its own workspace, act, y; the same fp32
    gradient buffers as the sparse step, counted again)."""
    T = a[0].shape[0]
    y = torch.empty((T, ffn.d), dtype=torch.float32, device="cuda")
    g = tuple(torch.empty_like(t) for t in grads)
    ws_before = ffn._ws.pop("ws", None)
    torch.cuda.synchronize()
    m0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    _, act = ffn.forward_train_dense(*a, y=y)
    ffn.backward_dense(*a, act, dy, out=g)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - m0 + sum(t.numel() * 4 for t in g) + T * ffn.d * 4

    def step():
        ffn.forward_train_dense(*a, y=y, act=act)
        ffn.backward_dense(*a, act, dy, out=g)

    steps_ms = []
    ms, _, _ = _timed(step, args.steps, args.warmup, torch, per_step=steps_ms)
    _, _, prof = _timed(step, args.steps, 0, torch, [ffn])
    ffn.check()
    flops = 2.0 * T * ffn.d * ffn.d_ff * (9 if ffn.gated else 6)
    if ws_before is not None:
        ffn._ws["ws"] = ws_before
    return {"kind": "this library's dense bf16 training step (sffn_forward_train_dense + "
                    "sffn_backward_dense)", "ms_per_step": ms, "value": T / ms,
            "step_ms": pct(steps_ms), "frac_of_mfma_peak": flops / (ms * 1e-3) / 1e12 /
            PEAK_BF16_TFLOPS, "kernels_ms_per_step": per_step(prof, args.steps),
            "act_bytes": int(act.numel() * 2), "peak_bytes": int(peak)}


def torch_dense_train(a, dy, steps, torch):
    """Context, not this library: torch's bf16 dense training step of the
    same layer (autograd through linear, relu, mul, linear; hipBLASLt
    GEMMs; bf16 gradients), its time per step and the device memory one
    step adds to the inputs and weights."""
    F_ = torch.nn.functional
    x = a[0].clone().requires_grad_()
    wg = a[1].clone().requires_grad_()
    wu = a[2].clone().requires_grad_()
    wdT = a[3].t().contiguous().requires_grad_()     # [d, F], the linear weight
    dyb = dy.clone()

    def step():
        h = F_.relu(F_.linear(x, wg)) * F_.linear(x, wu)
        yy = F_.linear(h, wdT)
        return torch.autograd.grad(yy, (x, wg, wu, wdT), dyb)

    step()
    torch.cuda.synchronize()
    m0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    h = F_.relu(F_.linear(x, wg)) * F_.linear(x, wu)
    yy = F_.linear(h, wdT)
    torch.cuda.synchronize()
    held = torch.cuda.memory_allocated() - m0
    g = torch.autograd.grad(yy, (x, wg, wu, wdT), dyb)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - m0
    del g, h, yy
    ms = _torch_ms(step, steps, torch)
    return {"kind": "torch autograd bf16 dense layer (not this library)", "ms_per_step": ms,
            "value": a[0].shape[0] / ms, "peak_bytes": int(peak),
            "after_forward_bytes": int(held)}


def bench_train(args, np, torch, SparseFFN, wl):
    import oracle
    W = wl.TRAIN_HYBRID
    inp = wl.make_inputs(W, seed=args.seed)
    n_cpu = (W.T if args.cpu_sample < 0 else min(args.cpu_sample, W.T))
    cpu_ms, cpu_runs = 0.0, 0
    if n_cpu > 0:
        # the oracle's training step: its float64 forward and backward
        x = inp.x[:n_cpu].astype(np.float64)
        wg = inp.w_gate.astype(np.float64).T
        wu = inp.w_up.astype(np.float64).T
        wd = inp.w_down.astype(np.float64)
        dy64 = inp.dy[:n_cpu].astype(np.float64)
        cpu_ms, cpu_runs = repeat_ms(lambda: oracle.backward(x, wg, wu, wd, dy64), CPU_MIN_MS)
        del x, wg, wu, wd, dy64
    a = [_dev(inp, k, torch, np) for k in ("x", "w_gate", "w_up", "w_down")]
    dy = _dev(inp, "dy", torch, np)
    del inp
    d, F, T = W.d, W.F, W.T
    # device memory the sparse step adds to its inputs and weights: the
    # Hybrid, the TwELL, y, the four gradients and the library's workspaces
    torch.cuda.synchronize()
    mem0 = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ffn = SparseFFN(d, F, gated=True, twell_cap=W.twell_cap, ell_cap=W.ell_cap,
                    dense_rows=W.dense_rows, dtype=torch.bfloat16, store_dtype=_store(args, torch))
    hy = ffn.new_hybrid(T)
    y = torch.empty((T, d), dtype=torch.float32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    grads = (torch.empty((T, d), **f32), torch.empty((F, d), **f32),
             torch.empty((F, d), **f32), torch.empty((F, d), **f32))

    # the TwELL of the step lives in the library's workspace (tw = None):
    # the backward needs only the Hybrid
    def step():
        ffn.forward_train(*a, hy=hy, y=y, check=False)
        ffn.backward(*a, hy, dy, out=grads)

    # one checked step first: the backup rows fit the Hybrid's capacity
    ffn.forward_train(*a, hy=hy, y=y)
    torch.cuda.synchronize()
    mem_fwd = torch.cuda.memory_allocated() - mem0
    ffn.backward(*a, hy, dy, out=grads)
    torch.cuda.synchronize()
    mem_sparse = torch.cuda.max_memory_allocated() - mem0
    mem_hybrid = sum(v.numel() * v.element_size() for v in hy.values()
                     if isinstance(v, torch.Tensor))
    mem_ws = ffn._ws["ws"].numel()
    mem_grads = sum(t.numel() * t.element_size() for t in grads)

    steps_ms = []
    ms, wall_ms, _ = _timed(step, args.steps, args.warmup, torch, per_step=steps_ms)
    ms_p, _, prof = _timed(step, args.steps, 0, torch, [ffn])
    torch.cuda.synchronize()
    ffn.check()
    dense_step = dense_train(ffn, a, dy, grads, args, torch)
    torch_step = torch_dense_train(a, dy, args.steps, torch)
    if ffn.hybrid_check(hy) != 0:
        raise RuntimeError("backup rows exceed the Hybrid's capacity")
    cnt = hy["ell_cnt"].cpu().numpy().astype(np.int64)
    slot = hy["slot"].cpu().numpy()[:T]
    nb = int(hy["n_backup"][0].item())
    P = int(cnt.sum())               # ELL slots (active pairs of ELL rows)
    R = int((slot < 0).sum())        # ELL rows
    S = args.steps
    # algorithmic bytes per step of the gather-bound kernels (bf16 operands,
    # sv bytes per stored activation value):
    # forward up/down: per slot W_u, W_d rows + (a, u, idx) saved; per row x, y
    sv = 2 if args.store == "bf16" else 4
    fwd = P * (2 * d * 2 + 2 * sv + 2) + R * (d * 2 + d * 4)
    # dH = dy . W_d[j] per slot: the W_d row and the index; per row the dy row
    sddmm = P * (d * 2 + 2) + R * d * 2
    # dx: per slot W_g, W_u rows, (idx, a, u, dh partial) in, (dZ, dU) out;
    # per row the dx row
    bdx = P * (2 * d * 2 + 2 + 2 * sv + 4 + 8) + R * d * 4
    # dW: per slot the x and dy rows and (dZ, dU, a, u, slot id); per neuron
    # its three dW rows
    bdw = P * (2 * d * 2 + 20) + F * 3 * d * 4
    rs = [roof("mfma", "gate_gemm_twell", 2.0 * T * d * F * S, prof, ["gate_gemm_twell"],
               PEAK_BF16_TFLOPS),
          roof("hbm", "sparse_up + sparse_hsum + sparse_down", fwd * S, prof,
               ["sparse_up", "sparse_hsum", "sparse_down"], PEAK_HBM_GBS),
          roof("hbm", "bwd_sddmm", sddmm * S, prof, ["bwd_sddmm"], PEAK_HBM_GBS),
          roof("hbm", "bwd_dx", bdx * S, prof, ["bwd_dx"], PEAK_HBM_GBS),
          roof("hbm", "bwd_dw", bdw * S, prof, ["bwd_dw"], PEAK_HBM_GBS)]
    rs = [r for r in rs if r is not None]
    ks = per_step(prof, S)
    rs.sort(key=lambda r: -r["avg_ms"] * r["launches"])
    out = {
        "metric": METRIC_TRAIN,
        "value": T / ms,
        "unit": "input tokens/ms",
        "n_gpus": 1,
        "steps": S,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": W.dtype,
        "data": "synthetic",
        "config": {"workload": W.name, "T": T, "d": d, "d_ff": F, "gated": True,
                   "nnz_per_token": W.nnz, "twell_cap": W.twell_cap, "ell_cap": W.ell_cap,
                   "dense_rows": W.dense_rows, "store_dtype": args.store,
                   "outlier_frac": W.outlier_frac, "seed": args.seed},
        "roofline": rs[0],
        "roofline_other": rs[1:],
        "dense_baseline": dict(dense_step, speedup_sparse_over_dense=
                               dense_step["ms_per_step"] / ms),
        "step_ms": pct(steps_ms),
        "torch_dense_train_step": dict(torch_step, speedup_sparse_over_torch_dense=
                                       torch_step["ms_per_step"] / ms),
        "peak_memory_bytes": {
            "sparse_step": int(mem_sparse),
            "sparse_saved_for_backward": int(mem_hybrid),
            "sparse_held_after_forward": int(mem_fwd),
            "sparse_workspace": int(mem_ws), "sparse_fp32_grads": int(mem_grads),
            "dense_step": dense_step["peak_bytes"],
            "dense_saved_for_backward": dense_step["act_bytes"],
            "torch_dense_step": torch_step["peak_bytes"],
            "torch_dense_held_after_forward": torch_step["after_forward_bytes"],
            "method": "torch.cuda.max_memory_allocated over one step (and memory_allocated "
                      "after the forward), less what the inputs and weights already held. "
                      "Sparse: the Hybrid (what the backward reads), y fp32, the four fp32 "
                      "gradients and the library's one workspace (TwELL inside it). Torch: "
                      "the autograd graph's saved tensors, y and its bf16 gradients"},
        "kernels_ms_per_step": ks,
        "ms_per_step_wall": wall_ms,
        "ms_per_step_with_kernel_events": ms_p,
        "backup_rows": nb,
        "ell_slots": P,
        "saved_activation_bytes": {
            "hybrid": int(T * W.ell_cap * (2 * sv + 2) + T * 8 + nb * (F * 2 * sv + 4)),
            "dense_a_u_fp32": int(T * F * 8)},
    }
    if n_cpu > 0:
        out["cpu_baseline"] = cpu_record(
            n_cpu * cpu_runs, cpu_ms,
            f"first {n_cpu} of {T} tokens, {cpu_runs} run(s): numpy float64 forward and "
            f"backward (the gradients of x and of all three weights)")
    return out


if __name__ == "__main__":
    sys.exit(main())
