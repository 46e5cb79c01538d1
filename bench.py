#!/usr/bin/env python3
"""Benchmark of one rank's tensor-parallel MLP shard on one MI355X.

Workload: the Llama-3-70B FFN shard (N = 4096 tokens, D = 8192, F = 28672 split T = 8 ways,
F/T = 3584; shard 0), bf16 inputs, fp32 accumulation, GELU (tanh form). One step is the
forward shard through the C ABI: the column-parallel up-projection with fused bias + GELU
(mlp_tp_up_proj) and the row-parallel down-projection to the fp32 partial (mlp_tp_down_proj).
`value` is the forward's GEMM work (4 N D F/T flops) per second.

Also measured in the same run, each over its own timed loop (reported under "rows"): the
same forward step with operands that are not in any cache (three copies in rotation), the
block-tail reduction of 8 fp32 partials [2048, 12288] with b2 (the GPT-3-175B layer's tail),
the shard backward at the Llama shape, the sum of 8 dX partials [4096, 8192], the gated
(SwiGLU) shard forward, the whole GPT-3-175B layer on one GPU with its tail as separate
partials + reduce, as an accumulating down-projection, and overlapped with the last shard's
down-projection, one token slice of that tail (reduce-scatter layout), and the shard forward
at the Llama shape for T = 1, 2, 4, 8.

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "TP-shard MLP fwd TFLOP/s + % bf16 MFMA peak (D=8192, F/T=3584, N=4096)"
WARMUP_MS = 250.0      # headline: from idle the clocks settle after ~40 ms of load
ROW_WARMUP_MS = 150.0  # each extra row, after its own input set-up

ROWS = ("fwd_cold_operands", "partial_reduce", "shard_bwd", "sum_dx", "gated_shard_fwd",
        "gated_shard_bwd", "gpt3_layer", "reduce_scatter_slice", "shard_count_sweep",
        "gpt2_medium_block", "epilogue_fusion_ablation", "small_products")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of every HIP source of the library: a counter record is valid only for these."""
    import glob
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tensor_mlp_block_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources (its recorded source hash matches); else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def read_profiled(kernel: str, workload: str, flop: float, sclk_live):
    """The committed kernel trace of the headline command (rocprofv3 --kernel-trace): the
    profiled run whose reported shader clock is nearest this run's, its rocprof mean duration
    of `kernel` over the timed steps, the fraction of peak that gives, and that fraction scaled
    by this run's clock over the profiled run's (throughput follows the clock the box runs at).
    `stale` is true when the kernel sources changed since the trace was taken."""
    path = os.path.join(ROOT, "profiles", f"kernel_trace_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    runs = [r for r in rec.get("runs", []) if kernel in r.get("kernels", {})]
    if not runs:
        return None
    best = min(runs, key=lambda r: abs((r.get("sclk_mhz") or 0) - (sclk_live or 0)))
    us = best["kernels"][kernel]["timed_avg_us"]
    frac = flop / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS
    out = {"source": f"profiles/kernel_trace_{workload}.txt", "runs": len(runs),
           "stale": rec.get("source_hash") != kernel_source_hash(),
           "rocprof_timed_avg_us": us, "frac": round(frac, 4), "sclk_mhz": best.get("sclk_mhz")}
    if sclk_live and best.get("sclk_mhz"):
        out["frac_scaled_to_this_sclk"] = round(frac * sclk_live / best["sclk_mhz"], 4)
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-ms", type=float, default=WARMUP_MS,
                    help="untimed warmup runs at least --warmup steps and at least this much "
                         "GPU time: from idle the GPU's clocks take ~40 ms of load to settle")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the extra per-row timings")
    ap.add_argument("--rows", default="all",
                    help="comma-separated subset of the extra rows to time: " + ", ".join(ROWS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle baseline sample")
    ap.add_argument("--cpu-row-seconds", type=float, default=3.0,
                    help="target CPU time of each sampled oracle timing of the other workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy three times, as the "
                         "known-size reference for hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the shard runs on one GPU; see the design notes for how it would shard).",
              file=sys.stderr)
        return 2

    import torch
    from tensor_mlp_block_amd import binding as mt
    from tensor_mlp_block_amd import synth, workloads

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    mt.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("[bench] calibration copy: 3 x 1 GiB read + 1 GiB write")
        del src, dst

    w = workloads.LLAMA70B_SHARD_T8
    N, D, F, T, Fs = w.N, w.D, w.F, w.T, w.Fs
    log(f"[bench] workload {w.name}: generating inputs")
    Xc = synth.gen_X(w)
    W1c, b1c, W2c = synth.gen_W1(w, 0, Fs), synth.gen_b1(w, 0, Fs), synth.gen_W2(w, 0, Fs)
    X, W1, b1, W2 = Xc.to(dev), W1c.to(dev), b1c.to(dev), W2c.to(dev)
    H = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
    P = torch.empty((N, D), dtype=torch.float32, device=dev)

    def step():
        mt.mlp_tp_up_proj(X, W1, b1, None, H, N, D, F, T, mt.BF16, w.act)
        mt.mlp_tp_down_proj(H, W2, P, N, D, F, T, mt.BF16)

    global ROW_WARMUP_MS
    ROW_WARMUP_MS = min(ROW_WARMUP_MS, args.warmup_ms)  # a shorter requested warmup applies to rows
    warm_steps, warm_ms = warm_up(torch, step, args.warmup, args.warmup_ms)
    log(f"[bench] warmup {warm_steps} steps, {warm_ms:.0f} ms")

    # Timed region: exactly K steps between two events, nothing else on the stream, so that
    # `value` holds the steps alone (each event recorded between launches adds a few
    # microseconds to the GPU timeline).
    K = args.steps
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(K):
        step()
    t1.record(stream)
    sclk_mhz = read_sclk_mhz(torch, dev)  # read while the timed steps run
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / K

    # Kernel durations for the roofline: a second pass of K steps with one event after every
    # launch (all on torch's current stream, which is the stream the binding launches on).
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * K + 1)]
    ev[0].record(stream)
    for i in range(K):
        mt.mlp_tp_up_proj(X, W1, b1, None, H, N, D, F, T, mt.BF16, w.act)
        ev[2 * i + 1].record(stream)
        mt.mlp_tp_down_proj(H, W2, P, N, D, F, T, mt.BF16)
        ev[2 * i + 2].record(stream)
    torch.cuda.synchronize()
    up_ms = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(K)]
    down_ms = [ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) for i in range(K)]
    step_ms = sorted(u + d for u, d in zip(up_ms, down_ms))
    median_ms = step_ms[K // 2] if K % 2 else 0.5 * (step_ms[K // 2 - 1] + step_ms[K // 2])
    gemm_flop = 2.0 * N * D * Fs
    fwd_flop = 2.0 * gemm_flop
    value = fwd_flop / (ms_per_step * 1e-3) / 1e12
    mean_up, mean_down = sum(up_ms) / K, sum(down_ms) / K
    log(f"[bench] step {ms_per_step:.4f} ms  {value:.1f} TFLOP/s | event pass: up {mean_up:.4f} ms  "
        f"down {mean_down:.4f} ms  step median {median_ms:.4f} ms")

    dominant = "up_proj" if mean_up >= mean_down else "down_proj"
    dom_ms = max(mean_up, mean_down)
    achieved = gemm_flop / (dom_ms * 1e-3) / 1e12
    kernel_name = {"up_proj": "gemm_up_proj_bias_gelu", "down_proj": "gemm_down_proj_f32"}[dominant]
    roofline = {
        "kernel": kernel_name,
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": read_traffic(kernel_name, w.name),
        "algorithmic_flop_per_launch": gemm_flop,
        "mean_launch_ms": round(dom_ms, 5),
        "other_kernel": {"name": ("gemm_down_proj_f32" if dominant == "up_proj"
                                  else "gemm_up_proj_bias_gelu"),
                         "mean_launch_ms": round(min(mean_up, mean_down), 5),
                         "achieved": round(gemm_flop / (min(mean_up, mean_down) * 1e-3) / 1e12, 2)},
    }

    roofline["profiled"] = read_profiled(kernel_name, w.name, gemm_flop, sclk_mhz)

    rows = None
    if not args.no_rows:
        want = ROWS if args.rows == "all" else tuple(r for r in args.rows.split(",") if r)
        unknown = [r for r in want if r not in ROWS]
        if unknown:
            log(f"unknown rows {unknown}; choose from {ROWS}")
            return 2
        rows = measure_rows(torch, mt, synth, workloads, dev, X, W1, b1, W2, H, w, want)

    cpu = None
    cpu_rows = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(Xc, W1c, b1c, W2c, w, args.cpu_seconds)
        cpu_rows = cpu_baseline_rows(synth, workloads, args.cpu_row_seconds)

    props = torch.cuda.get_device_properties(dev)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warm_steps,
        "warmup_ms": round(warm_ms, 1),
        "ms_per_step": round(ms_per_step, 5),
        "event_pass": {"ms_per_step_median": round(median_ms, 5),
                       "ms_per_step_min": round(step_ms[0], 5),
                       "up_ms_mean": round(mean_up, 5), "down_ms_mean": round(mean_down, 5)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": w.name, "N": N, "D": D, "F": F, "T": T, "Fs": Fs, "shard": 0,
                   "act": w.act, "parallelism": "one rank's shard on 1 GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_rows": cpu_rows,
        "rows": rows,
        "device": torch.cuda.get_device_name(dev),
        "arch": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "sclk_mhz_during_timing": sclk_mhz,
        # value over the dense bf16 rate at the clock the driver reported during the timed steps
        # (CUs x 4096 FLOP/clock x sclk): context for box-to-box clock spread, not the roofline.
        "pct_of_peak_at_reported_sclk": (round(100.0 * value / (props.multi_processor_count * 4096.0
                                                                  * sclk_mhz * 1e-6), 2)
                                         if sclk_mhz else None),
        "hip": getattr(torch.version, "hip", None),
    }
    print(json.dumps(out), flush=True)
    return 0


def read_sclk_mhz(torch, dev):
    """The shader clock the driver reports for this GPU (the DPM level marked '*'), or None.
    The DRM card is matched to the device by its PCI address."""
    import glob
    props = torch.cuda.get_device_properties(dev)
    bus, domain = getattr(props, "pci_bus_id", None), getattr(props, "pci_domain_id", None)
    if bus is None:
        return None
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            addr = os.path.basename(os.path.realpath(os.path.dirname(path)))  # "0000:75:00.0"
            dom, b = addr.split(":")[:2]
            if int(b, 16) != bus or (domain is not None and int(dom, 16) != domain):
                continue
            with open(path) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        return int(line.split(":")[1].strip().lower().split("mhz")[0])
        except (OSError, ValueError, IndexError):
            continue
    return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def warm_up(torch, fn, min_calls, min_ms, chunk=8):
    """Runs fn at least `min_calls` times and for at least `min_ms` of GPU time, untimed.

    From idle, the GPU's clocks ramp up over the first ~40 ms of sustained load (a 50 ms pause
    is enough to drop them again), so a fixed handful of warmup calls leaves the timed region
    inside the ramp. Calls are issued in chunks with at most two chunks in flight, so the GPU
    never idles while the host checks the elapsed time. Returns (calls, GPU ms)."""
    s = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t0.record(s)
    calls, pending = 0, None
    while True:
        for _ in range(chunk):
            fn()
        calls += chunk
        ev = torch.cuda.Event(enable_timing=True)
        ev.record(s)
        if pending is not None:
            pending.synchronize()
            if calls - chunk >= min_calls and t0.elapsed_time(pending) >= min_ms:
                break
        pending = ev
    torch.cuda.synchronize()
    return calls, t0.elapsed_time(ev)


def _time_loop(torch, fn, iters, warm_ms=None):
    warm_up(torch, fn, 3, ROW_WARMUP_MS if warm_ms is None else warm_ms)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    s = torch.cuda.current_stream()
    a.record(s)
    for _ in range(iters):
        fn()
    b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def measure_rows(torch, mt, synth, workloads, dev, X, W1, b1, W2, H, w, want=ROWS):
    res = {}
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    if "fwd_cold_operands" in want:
        res.update(_row_cold(torch, mt, dev, X, W1, b1, W2, H, w))
    if "epilogue_fusion_ablation" in want:
        res.update(_row_fusion_ablation(torch, mt, dev, X, W1, b1, H, w))
    if "partial_reduce" in want:
        res.update(_row_partial_reduce(torch, mt, synth, workloads, dev, g))
    if "shard_bwd" in want or "sum_dx" in want:
        res.update(_rows_backward(torch, mt, synth, workloads, dev, g, X, W1, b1, W2, want))
    res.update(measure_next_rows(torch, mt, synth, workloads, dev, g, want))
    return res


def _row_cold(torch, mt, dev, X, W1, b1, W2, H, w, copies=3):
    """The headline step with operands that are not in any cache: the steps rotate through
    `copies` separate copies of X, W1, b1, W2 (together larger than the 256 MB last-level cache),
    so each step reads its operands from HBM. The headline itself repeats one set of operands,
    which then stays in that cache from step to step."""
    N, D, F, T, Fs = w.N, w.D, w.F, w.T, w.Fs
    sets = [(X, W1, b1, W2)] + [(X.clone(), W1.clone(), b1.clone(), W2.clone())
                                for _ in range(copies - 1)]
    P = torch.empty((N, D), dtype=torch.float32, device=dev)
    steps = 10 * copies
    s = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    turn = [0]

    def rotating_step():
        Xi, W1i, b1i, W2i = sets[turn[0] % copies]
        turn[0] += 1
        mt.mlp_tp_up_proj(Xi, W1i, b1i, None, H, N, D, F, T, mt.BF16, w.act)
        mt.mlp_tp_down_proj(H, W2i, P, N, D, F, T, mt.BF16)

    warm_up(torch, rotating_step, 2 * copies, ROW_WARMUP_MS)
    for i in range(steps):
        Xi, W1i, b1i, W2i = sets[i % copies]
        ev[i][0].record(s)
        mt.mlp_tp_up_proj(Xi, W1i, b1i, None, H, N, D, F, T, mt.BF16, w.act)
        ev[i][1].record(s)
        mt.mlp_tp_down_proj(H, W2i, P, N, D, F, T, mt.BF16)
        ev[i][2].record(s)
    torch.cuda.synchronize()
    up = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    down = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    flop = 4.0 * N * D * Fs
    out = {"copies": copies, "up_ms": round(up, 5), "down_ms": round(down, 5),
           "TFLOP/s": round(flop / ((up + down) * 1e-3) / 1e12, 1),
           "frac_mfma": round(flop / ((up + down) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    log(f"[bench] forward with cold operands: up {up:.4f} ms down {down:.4f} ms, "
        f"{out['TFLOP/s']} TFLOP/s")
    del sets, P
    return {"fwd_cold_operands": out}


def _row_fusion_ablation(torch, mt, dev, X, W1, b1, H, w):
    """What fusing bias + GELU into the up-projection's GEMM saves: the fused launch against the
    same GEMM writing its fp32 result, then the epilogue as a kernel of its own (which reads that
    result back from HBM and writes H)."""
    N, D, F, T, Fs = w.N, w.D, w.F, w.T, w.Fs
    Z32 = torch.empty((N, Fs), device=dev)

    def fused():
        mt.mlp_tp_up_proj(X, W1, b1, None, H, N, D, F, T, mt.BF16, w.act)

    def gemm_only():
        # P[N, D'] = X[N, F'] W1^(r)[F', D'] with D' = Fs, F' = D, T' = 1: the up-projection's
        # product, written as fp32
        mt.mlp_tp_down_proj(X, W1, Z32, N, Fs, D, 1, mt.BF16)

    def epilogue_only():
        mt.mlp_tp_bias_act(Z32, b1, H, N, F, T, mt.BF16, w.act)

    ms_f = _time_loop(torch, fused, 50)
    ms_g = _time_loop(torch, gemm_only, 50)
    ms_e = _time_loop(torch, epilogue_only, 50)
    ep_bytes = N * Fs * (4 + 2) + Fs * 2
    flop = 2.0 * N * D * Fs
    out = {"workload": w.name, "fused_ms": round(ms_f, 5), "gemm_fp32_out_ms": round(ms_g, 5),
           "standalone_epilogue_ms": round(ms_e, 5), "unfused_ms": round(ms_g + ms_e, 5),
           "fused_TFLOP/s": round(flop / (ms_f * 1e-3) / 1e12, 1),
           "unfused_TFLOP/s": round(flop / ((ms_g + ms_e) * 1e-3) / 1e12, 1),
           "standalone_epilogue_GB/s": round(ep_bytes / (ms_e * 1e-3) / 1e9, 1),
           "standalone_epilogue_frac_hbm": round(ep_bytes / (ms_e * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "standalone_epilogue_bytes": ep_bytes}
    log(f"[bench] epilogue fusion: fused {ms_f:.4f} ms | GEMM to fp32 {ms_g:.4f} + epilogue "
        f"{ms_e:.4f} ms ({out['standalone_epilogue_GB/s']} GB/s)")
    del Z32
    return {"epilogue_fusion_ablation": out}


def _row_partial_reduce(torch, mt, synth, workloads, dev, g):
    res = {}
    # Block tail of the GPT-3-175B layer: 8 fp32 partials [2048, 12288] + bf16 b2, once.
    w4 = workloads.GPT3_175B_T8
    parts = [torch.randn((w4.N, w4.D), generator=g, device=dev) for _ in range(w4.T)]
    b2 = synth.gen_b2(w4).to(dev)
    Y = torch.empty((w4.N, w4.D), device=dev)
    ms = _time_loop(torch, lambda: mt.mlp_tp_partial_reduce(parts, w4.T, b2, mt.BF16, Y, w4.N,
                                                            w4.D), 20)
    nbytes = (w4.T + 1) * 4.0 * w4.N * w4.D + 2.0 * w4.D
    res["partial_reduce"] = {"workload": w4.name, "T": w4.T, "ms": round(ms, 5),
                             "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                             "algorithmic_bytes": nbytes}
    log(f"[bench] reduce T=8 [2048,12288]: {ms:.4f} ms, {res['partial_reduce']['GB/s']} GB/s")
    del parts, Y
    return res


def _rows_backward(torch, mt, synth, workloads, dev, g, X, W1, b1, W2, want):
    res = {}
    # Backward of the Llama shard (dY ~ N(0,1), seed 505).
    w5 = workloads.LLAMA70B_SHARD_T8_BWD
    N, D, F, T, Fs = w5.N, w5.D, w5.F, w5.T, w5.Fs
    dY = synth.gen_dY(w5).to(dev)
    Z = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
    Hz = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
    P = torch.empty((N, D), device=dev)
    mt.mlp_tp_shard_fwd(X, W1, b1, W2, Hz, Z, P, N, D, F, T, mt.BF16, w5.act)
    dZ = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
    dW1 = torch.empty((D, Fs), device=dev)
    dW2 = torch.empty((Fs, D), device=dev)
    db1 = torch.empty((Fs,), device=dev)
    dX = torch.empty((N, D), device=dev)
    nb = mt.mlp_tp_shard_bwd_workspace_bytes(N, D, F, T)
    ws = torch.empty((nb,), dtype=torch.uint8, device=dev)
    if "shard_bwd" in want:
        ms = _time_loop(torch, lambda: mt.mlp_tp_shard_bwd(X, W1, W2, Z, Hz, dY, dZ, dW1, db1,
                                                           dW2, dX, ws, nb, N, D, F, T, mt.BF16,
                                                           w5.act), 10)
        flop = 8.0 * N * D * Fs
        res["shard_bwd"] = {"workload": w5.name, "ms": round(ms, 5),
                            "TFLOP/s": round(flop / (ms * 1e-3) / 1e12, 1),
                            "frac_mfma": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] shard bwd: {ms:.4f} ms, {res['shard_bwd']['TFLOP/s']} TFLOP/s")
    del dZ, dW1, dW2, db1, Z, Hz, P
    if "sum_dx" not in want:
        return res

    # Sum of the 8 dX partials [4096, 8192] (no bias).
    parts = [torch.randn((N, D), generator=g, device=dev) for _ in range(T)]
    ms = _time_loop(torch, lambda: mt.mlp_tp_partial_reduce(parts, T, None, mt.F32, dX, N, D), 20)
    nbytes = (T + 1) * 4.0 * N * D
    res["sum_dx"] = {"workload": w5.name, "T": T, "ms": round(ms, 5),
                     "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                     "algorithmic_bytes": nbytes}
    log(f"[bench] sum dX T=8 [4096,8192]: {ms:.4f} ms, {res['sum_dx']['GB/s']} GB/s")
    del parts, dX, dY, ws
    return res


def _randn_bf16(torch, shape, std, g, dev):
    return (torch.randn(shape, generator=g, device=dev) * std).to(torch.bfloat16)


def measure_next_rows(torch, mt, synth, workloads, dev, g, want=ROWS):
    """The gated shard, the three forms of the GPT-3-175B layer's block tail, one token slice of
    that tail, and the shard-count sweep at the Llama shape. Weights for these timing rows are
    drawn on the GPU (torch.randn, the workloads' distributions); parity is the tests' job."""
    res = {}
    if "gated_shard_fwd" in want or "gated_shard_bwd" in want:
        res.update(_row_gated(torch, mt, workloads, dev, g, want))
    if "gpt3_layer" in want or "reduce_scatter_slice" in want:
        res.update(_rows_gpt3_layer(torch, mt, workloads, dev, g, want))
    if "shard_count_sweep" in want:
        res.update(_row_t_sweep(torch, mt, workloads, dev, g))
    if "gpt2_medium_block" in want:
        res.update(_row_gpt2_medium(torch, mt, workloads, dev, g))
    if "small_products" in want:
        res.update(_row_small_products(torch, mt, workloads, dev, g))
    return res


def _row_small_products(torch, mt, workloads, dev, g):
    """Shards whose products have too few output tiles to fill the GPU: the pages' example shape
    (256 tokens, D 4096, F 11008) at T = 1, 2, 4, 8 and one GPT-2-medium shard (4096 tokens, D
    1024, F 4096, T 2), each as mlp_tp_shard_fwd and as mlp_tp_shard_fwd_ws with the workspace
    its query asks for (products with at most half the 128 x 128 workgroup slots filled split
    their contraction)."""
    cases = [(workloads.PAGE_EXAMPLE_MLP.with_(T=T), f"page_example_t{T}") for T in (1, 2, 4, 8)]
    cases.append((workloads.GPT2_MEDIUM_T2, "gpt2_medium_shard"))
    out = {}
    for w, key in cases:
        N, D, F, T, Fs = w.N, w.D, w.F, w.T, w.Fs
        X = _randn_bf16(torch, (N, D), 1.0, g, dev)
        W1 = _randn_bf16(torch, (D, Fs), 0.02, g, dev)
        b1 = _randn_bf16(torch, (Fs,), 0.02, g, dev)
        W2 = _randn_bf16(torch, (Fs, D), 0.02, g, dev)
        H = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
        P = torch.empty((N, D), device=dev)
        nb = mt.mlp_tp_shard_fwd_workspace_bytes(N, D, F, T)
        ws = torch.empty((max(nb, 16),), dtype=torch.uint8, device=dev)
        plain = _time_loop(torch, lambda: mt.mlp_tp_shard_fwd(X, W1, b1, W2, H, None, P, N, D, F,
                                                              T, mt.BF16, w.act), 50)
        split = _time_loop(torch, lambda: mt.mlp_tp_shard_fwd_ws(X, W1, b1, W2, H, None, P, ws, nb,
                                                                 N, D, F, T, mt.BF16, w.act), 50)
        flop = 4.0 * N * D * Fs
        tiles = {p: mt.mlp_tp_shard_tile(p, N, D, F, T, torch.cuda.get_device_properties(dev)
                                         .multi_processor_count)[:2] for p in ("up", "down")}
        out[key] = {"N": N, "D": D, "F": F, "T": T, "tiles": tiles, "workspace_bytes": nb,
                    "ms": round(plain, 5), "TFLOP/s": round(flop / (plain * 1e-3) / 1e12, 1),
                    "split_ms": round(split, 5),
                    "split_TFLOP/s": round(flop / (split * 1e-3) / 1e12, 1)}
        log(f"[bench] small products {key}: {plain:.4f} ms unsplit, {split:.4f} ms with "
            f"{nb / 1e6:.1f} MB of workspace")
        del X, W1, b1, W2, H, P, ws
    return {"small_products": out}


def _row_gpt2_medium(torch, mt, workloads, dev, g):
    """The GPT-2-medium-shaped block (N=4096, D=1024, F=4096, T=2) on one GPU: both shards'
    forward, then the 2-way tail with b2. Its products are too small for the 256-wide tiles to
    fill the GPU, so they take the 128 x 128 tile. Timed two ways: the shards one after the other
    on one stream, and the two shards on two streams (as two ranks would run them), joined
    before the tail."""
    w = workloads.GPT2_MEDIUM_T2
    N, D, F, T, Fs = w.N, w.D, w.F, w.T, w.Fs
    X = _randn_bf16(torch, (N, D), 1.0, g, dev)
    W1s = [_randn_bf16(torch, (D, Fs), 0.02, g, dev) for _ in range(T)]
    b1s = [_randn_bf16(torch, (Fs,), 0.02, g, dev) for _ in range(T)]
    W2s = [_randn_bf16(torch, (Fs, D), 0.02, g, dev) for _ in range(T)]
    b2 = _randn_bf16(torch, (D,), 0.02, g, dev)
    Hs = [torch.empty((N, Fs), dtype=torch.bfloat16, device=dev) for _ in range(T)]
    parts = [torch.empty((N, D), device=dev) for _ in range(T)]
    Y = torch.empty((N, D), device=dev)
    main = torch.cuda.current_stream()
    side = [torch.cuda.Stream() for _ in range(T - 1)]  # default priority
    fork = [torch.cuda.Event() for _ in range(T - 1)]
    join = [torch.cuda.Event() for _ in range(T - 1)]

    def block_one_stream():
        for r in range(T):
            mt.mlp_tp_shard_fwd(X, W1s[r], b1s[r], W2s[r], Hs[r], None, parts[r], N, D, F, T,
                                mt.BF16, w.act)
        mt.mlp_tp_partial_reduce(parts, T, b2, mt.BF16, Y, N, D)

    def block_streams():
        for r in range(1, T):
            fork[r - 1].record(main)
            side[r - 1].wait_event(fork[r - 1])
            mt.mlp_tp_shard_fwd(X, W1s[r], b1s[r], W2s[r], Hs[r], None, parts[r], N, D, F, T,
                                mt.BF16, w.act, stream=side[r - 1])
            join[r - 1].record(side[r - 1])
        mt.mlp_tp_shard_fwd(X, W1s[0], b1s[0], W2s[0], Hs[0], None, parts[0], N, D, F, T, mt.BF16,
                            w.act, stream=main)
        for e in join:
            main.wait_event(e)
        mt.mlp_tp_partial_reduce(parts, T, b2, mt.BF16, Y, N, D)

    ms1 = _time_loop(torch, block_one_stream, 50)
    ms = _time_loop(torch, block_streams, 50)
    flop = 4.0 * N * D * F
    tf = lambda t: round(flop / (t * 1e-3) / 1e12, 1)
    out = {"workload": w.name, "ms": round(ms, 5), "TFLOP/s": tf(ms),
           "frac_mfma": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "streams": T,
           "one_stream_ms": round(ms1, 5), "one_stream_TFLOP/s": tf(ms1)}
    log(f"[bench] gpt2-medium block (2 shards + tail): {ms:.4f} ms, {out['TFLOP/s']} TFLOP/s on "
        f"{T} streams; one stream {ms1:.4f} ms")
    del X, W1s, b1s, W2s, b2, Hs, parts, Y
    return {"gpt2_medium_block": out}


def _row_gated(torch, mt, workloads, dev, g, want):
    res = {}
    # Gated (SwiGLU) shard of the Llama-3-70B FFN: gate and up in one dual GEMM, then down; its
    # backward: dG and dU from one GEMM with the product rule in the epilogue, three weight
    # gradients, and dX as two GEMMs into one fp32 buffer.
    w = workloads.LLAMA70B_SWIGLU_SHARD_T8
    N, D, F, T, Fs = w.N, w.D, w.F, w.T, w.Fs
    X = _randn_bf16(torch, (N, D), 1.0, g, dev)
    Wg, Wu = _randn_bf16(torch, (D, Fs), 0.02, g, dev), _randn_bf16(torch, (D, Fs), 0.02, g, dev)
    W2 = _randn_bf16(torch, (Fs, D), 0.02, g, dev)
    H = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
    P = torch.empty((N, D), device=dev)
    if "gated_shard_fwd" in want:
        ms = _time_loop(torch, lambda: mt.mlp_tp_swiglu_shard_fwd(X, Wg, Wu, W2, None, None, H, P,
                                                                  N, D, F, T, mt.BF16), 20)
        flop = 6.0 * N * D * Fs
        res["gated_shard_fwd"] = {"workload": w.name, "ms": round(ms, 5),
                                  "TFLOP/s": round(flop / (ms * 1e-3) / 1e12, 1),
                                  "frac_mfma": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                                     4)}
        log(f"[bench] gated shard fwd: {ms:.4f} ms, {res['gated_shard_fwd']['TFLOP/s']} TFLOP/s")
    if "gated_shard_bwd" in want:
        G = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
        U = torch.empty_like(G)
        mt.mlp_tp_swiglu_shard_fwd(X, Wg, Wu, W2, G, U, H, P, N, D, F, T, mt.BF16)
        dY = torch.randn((N, D), generator=g, device=dev).to(torch.bfloat16)
        dG, dU = torch.empty_like(G), torch.empty_like(G)
        dWg, dWu = torch.empty((D, Fs), device=dev), torch.empty((D, Fs), device=dev)
        dW2 = torch.empty((Fs, D), device=dev)
        dX = P  # the forward's partial buffer, reused
        ms = _time_loop(torch, lambda: mt.mlp_tp_swiglu_shard_bwd(
            X, Wg, Wu, W2, G, U, H, dY, dG, dU, dWg, dWu, dW2, dX, N, D, F, T, mt.BF16), 10)
        flop = 12.0 * N * D * Fs
        res["gated_shard_bwd"] = {"workload": w.name, "ms": round(ms, 5),
                                  "TFLOP/s": round(flop / (ms * 1e-3) / 1e12, 1),
                                  "frac_mfma": round(flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                                                     4)}
        log(f"[bench] gated shard bwd: {ms:.4f} ms, {res['gated_shard_bwd']['TFLOP/s']} TFLOP/s")
        del G, U, dY, dG, dU, dWg, dWu, dW2, dX
    del X, Wg, Wu, W2, H, P
    return res


def _rows_gpt3_layer(torch, mt, workloads, dev, g, want):
    res = {}
    # The GPT-3-175B MLP layer on one GPU: 8 shards of F/T = 6144 in sequence and the tail,
    #   separate: 8 fp32 partials, then the T-way reduce with b2;
    #   accumulate: each down-projection adds into one buffer seeded with b2;
    #   overlapped: shards 0-6 as in `separate`, shard 7's down-projection in token chunks with
    #   each finished chunk's tail on a second stream.
    w = workloads.GPT3_175B_T8
    N, D, F, T, Fs = w.N, w.D, w.F, w.T, w.Fs
    X = _randn_bf16(torch, (N, D), 1.0, g, dev)
    W1s = [_randn_bf16(torch, (D, Fs), 0.02, g, dev) for _ in range(T)]
    b1s = [_randn_bf16(torch, (Fs,), 0.02, g, dev) for _ in range(T)]
    W2s = [_randn_bf16(torch, (Fs, D), 0.02, g, dev) for _ in range(T)]
    b2 = _randn_bf16(torch, (D,), 0.02, g, dev)
    b2f = b2.float()
    H = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
    parts = [torch.empty((N, D), device=dev) for _ in range(T)]
    Y = torch.empty((N, D), device=dev)
    side = torch.cuda.Stream(device=dev)
    chunk = 1024  # two chunks: each chunk's GEMM still fills most of the CUs

    def separate():
        for r in range(T):
            mt.mlp_tp_shard_fwd(X, W1s[r], b1s[r], W2s[r], H, None, parts[r], N, D, F, T, mt.BF16,
                                w.act)
        mt.mlp_tp_partial_reduce(parts, T, b2, mt.BF16, Y, N, D)

    def accumulate():
        Y.copy_(b2f.expand(N, D))
        for r in range(T):
            mt.mlp_tp_up_proj(X, W1s[r], b1s[r], None, H, N, D, F, T, mt.BF16, w.act)
            mt.mlp_tp_down_proj_accumulate(H, W2s[r], Y, N, D, F, T, mt.BF16)

    def overlapped():
        for r in range(T - 1):
            mt.mlp_tp_shard_fwd(X, W1s[r], b1s[r], W2s[r], H, None, parts[r], N, D, F, T, mt.BF16,
                                w.act)
        mt.mlp_tp_up_proj(X, W1s[T - 1], b1s[T - 1], None, H, N, D, F, T, mt.BF16, w.act)
        mt.mlp_tp_down_proj_overlap_tail(H, W2s[T - 1], parts, T, T - 1, b2, mt.BF16, Y, N, D, F,
                                         mt.BF16, chunk, tail_stream=side)

    flop = 4.0 * N * D * F  # all 8 shards' GEMMs
    if "gpt3_layer" in want:
        layer = {"workload": w.name, "flop": flop, "tail_chunk_rows": chunk}
        for name, fn in (("separate", separate), ("accumulate", accumulate),
                         ("overlapped", overlapped)):
            ms = _time_loop(torch, fn, 10)
            layer[name] = {"ms": round(ms, 4), "TFLOP/s": round(flop / (ms * 1e-3) / 1e12, 1)}
            log(f"[bench] gpt3 layer ({name}): {ms:.4f} ms")
        res["gpt3_layer"] = layer
    else:
        separate()  # the partials the slice reduces

    if "reduce_scatter_slice" not in want:
        return res
    # One token slice of that tail (reduce-scatter layout): rank 0's N / T rows.
    row0, rows = mt.mlp_tp_token_slice(N, T, 0)
    Yr = torch.empty((rows, D), device=dev)
    ms = _time_loop(torch, lambda: mt.mlp_tp_partial_reduce_scatter(parts, T, 0, b2, mt.BF16, Yr,
                                                                    N, D), 20)
    nbytes = (T + 1) * 4.0 * rows * D + 2.0 * D
    res["reduce_scatter_slice"] = {"workload": w.name, "T": T, "rows": rows, "ms": round(ms, 5),
                                   "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                   "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                   "algorithmic_bytes": nbytes}
    log(f"[bench] reduce-scatter slice: {ms:.4f} ms, {res['reduce_scatter_slice']['GB/s']} GB/s")
    del X, W1s, b1s, W2s, H, parts, Y, Yr
    return res


def _row_t_sweep(torch, mt, workloads, dev, g):
    res = {}
    # Shard count sweep at the Llama shape: one rank's forward for T = 1, 2, 4, 8.
    w = workloads.LLAMA70B_SHARD_T8
    N, D, F = w.N, w.D, w.F
    X = _randn_bf16(torch, (N, D), 1.0, g, dev)
    sweep = {}
    for T in (1, 2, 4, 8):
        Fs = F // T
        W1 = _randn_bf16(torch, (D, Fs), 0.02, g, dev)
        b1 = _randn_bf16(torch, (Fs,), 0.02, g, dev)
        W2 = _randn_bf16(torch, (Fs, D), 0.02, g, dev)
        H = torch.empty((N, Fs), dtype=torch.bfloat16, device=dev)
        P = torch.empty((N, D), device=dev)
        ms = _time_loop(torch, lambda: mt.mlp_tp_shard_fwd(X, W1, b1, W2, H, None, P, N, D, F, T,
                                                           mt.BF16, w.act), 10)
        tf = 4.0 * N * D * Fs / (ms * 1e-3) / 1e12
        sweep[str(T)] = {"Fs": Fs, "ms": round(ms, 4), "TFLOP/s": round(tf, 1)}
        log(f"[bench] T={T} shard fwd: {ms:.4f} ms, {tf:.1f} TFLOP/s")
        del W1, b1, W2, H, P
    res["shard_count_sweep"] = {"workload": w.name, "by_T": sweep}
    return res


def cpu_baseline(Xc, W1c, b1c, W2c, w, seconds):
    """The fp64 oracle, as it stands, on a bounded sample of token rows of the same shard."""
    import numpy as np
    import oracle

    W1, b1, W2 = (t.double().numpy() for t in (W1c, b1c, W2c))
    X = Xc.double().numpy()
    per_row_flop = 4.0 * w.D * w.Fs
    # Calibrate on one row per oracle thread (the oracle spreads rows over its threads).
    cal = max(2, min(w.N, oracle.num_threads()))
    t = time.perf_counter()
    oracle.shard_fwd(X[:cal], W1, b1, W2, 1, 0, act=w.act)
    dt = (time.perf_counter() - t) / cal
    rows = int(max(cal, min(w.N, seconds / max(dt, 1e-6))))
    idx = np.linspace(0, w.N - 1, rows).astype(np.int64)
    log(f"[bench] cpu baseline: {rows} rows (~{rows * dt:.1f} s)")
    t = time.perf_counter()
    oracle.shard_fwd(X[idx], W1, b1, W2, 1, 0, act=w.act)
    el = time.perf_counter() - t
    tflops = rows * per_row_flop / el / 1e12
    return {"value": round(tflops, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": round(el, 2), "cpu_model": cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"{rows} of {w.N} token rows of the {w.name} shard-0 forward "
                      f"(fp64 C oracle, OpenMP over rows)"}


def _oracle_rows_sample(run, N, seconds):
    """Times run(idx) on a bounded, evenly spread sample of token rows: a calibration call on
    one row per oracle thread sets the sample size for about `seconds` of CPU time. Returns
    (rows, elapsed seconds)."""
    import numpy as np
    import oracle

    cal = max(2, min(N, oracle.num_threads()))
    t = time.perf_counter()
    run(np.arange(cal))
    dt = (time.perf_counter() - t) / cal
    rows = int(max(cal, min(N, seconds / max(dt, 1e-6))))
    idx = np.linspace(0, N - 1, rows).astype(np.int64)
    t = time.perf_counter()
    run(idx)
    return rows, time.perf_counter() - t


def cpu_baseline_rows(synth, workloads, seconds):
    """The fp64 oracle, as it stands, timed on the other workloads: the GPT-2-medium block (both
    shards and the tail, whole), one GPT-3-175B shard's forward and the Llama shard's backward
    (token-row samples: every product's cost is linear in the rows), and the sum of 8 dX
    partials (a row sample). Reported beside the GPU rows; not a target."""
    import numpy as np
    import oracle

    out = {"cores": oracle.num_threads(), "kind": "oracle"}
    # GPT-2-medium block: 2 shards + tail, all 4096 rows.
    w = workloads.GPT2_MEDIUM_T2
    X = synth.gen_X(w).double().numpy()
    W1, b1, W2 = (t.double().numpy() for t in (synth.gen_W1(w), synth.gen_b1(w), synth.gen_W2(w)))
    b2 = synth.gen_b2(w).double().numpy()
    t = time.perf_counter()
    oracle.block_fwd(X, W1, b1, W2, b2, w.T, act=w.act)
    el = time.perf_counter() - t
    flop = 4.0 * w.N * w.D * w.F
    out["gpt2_medium_block"] = {"workload": w.name, "seconds": round(el, 2),
                                "TFLOP/s": round(flop / el / 1e12, 6),
                                "sample": "all 4096 token rows, both shards and the tail"}
    log(f"[bench] cpu rows: gpt2 block {el:.2f} s")
    # GPT-3-175B: shard 0's forward on a row sample.
    w = workloads.GPT3_175B_T8
    Fs = w.Fs
    X = synth.gen_X(w).double().numpy()
    W1, b1, W2 = (t.double().numpy() for t in (synth.gen_W1(w, 0, Fs), synth.gen_b1(w, 0, Fs),
                                               synth.gen_W2(w, 0, Fs)))
    rows, el = _oracle_rows_sample(lambda idx: oracle.shard_fwd(X[idx], W1, b1, W2, 1, 0,
                                                                act=w.act), w.N, seconds)
    out["gpt3_175b_shard_fwd"] = {"workload": w.name, "seconds": round(el, 2),
                                  "TFLOP/s": round(rows * 4.0 * w.D * Fs / el / 1e12, 6),
                                  "sample": f"{rows} of {w.N} token rows of shard 0's forward"}
    log(f"[bench] cpu rows: gpt3 shard {rows} rows {el:.2f} s")
    # Llama shard backward (dZ, dW1, db1, dW2, dX of shard 0) on a row sample.
    w = workloads.LLAMA70B_SHARD_T8_BWD
    Fs = w.Fs
    X = synth.gen_X(w).double().numpy()
    dY = synth.gen_dY(w).double().numpy()
    W1, b1, W2 = (t.double().numpy() for t in (synth.gen_W1(w, 0, Fs), synth.gen_b1(w, 0, Fs),
                                               synth.gen_W2(w, 0, Fs)))
    rows, el = _oracle_rows_sample(lambda idx: oracle.shard_bwd(X[idx], W1, b1, W2, dY[idx], 1, 0,
                                                                act=w.act), w.N, seconds)
    out["llama3_70b_shard_bwd"] = {"workload": w.name, "seconds": round(el, 2),
                                   "TFLOP/s": round(rows * 8.0 * w.D * Fs / el / 1e12, 6),
                                   "sample": f"{rows} of {w.N} token rows of shard 0's backward "
                                             "(the forward it needs is recomputed inside and not "
                                             "counted)"}
    log(f"[bench] cpu rows: llama bwd {rows} rows {el:.2f} s")
    # Sum of 8 dX partials [4096, 8192] fp32, on a row sample.
    rng = np.random.default_rng(505)
    nr = 512
    parts = [rng.standard_normal((nr, w.D)).astype(np.float32) for _ in range(8)]
    t = time.perf_counter()
    oracle.partial_sum(parts)
    el = time.perf_counter() - t
    out["sum_dx"] = {"workload": w.name, "seconds": round(el, 4),
                     "GB/s": round(9 * nr * w.D * 4 / el / 1e9, 2),
                     "sample": f"{nr} of {w.N} rows of the 8 fp32 partials"}
    return out


if __name__ == "__main__":
    sys.exit(main())
