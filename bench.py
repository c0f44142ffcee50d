#!/usr/bin/env python3
"""Throughput of the bf16 GEMM hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--workload NAME] [--graph]

A step is one call of the fused operation on one batch of synthetic input
already resident in device memory (default: linear + bias + GELU(tanh) at
M = N = K = 8192, W stored [N][K]).  Prints ONE JSON line with the throughput
in TFLOP/s (2*M*N*K flops per GEMM) over K timed steps, a roofline object for
the GEMM kernel (achieved TFLOP/s from HIP events around every launch on the
launch stream, in a second pass of the same number of launches after the
timed region, against the bf16 dense MFMA peak) and the CPU oracle's
throughput on a bounded sample of the same workload, timed on this host's
cores.

Settling.  After idle the GPU's clock ramps up over the first few tens of
milliseconds of work: at 8192^3, launches 5-25 after two idle seconds took
786 us on average (max 926), launches 25-45 715 us, and from about launch 45
on 693-697 us, flat to launch 3000.  So the W warm-up launches are followed,
when they are fewer, by more untimed launches until at least SETTLE_LAUNCHES
launches and SETTLE_SECONDS of launches have run; the JSON line reports that
settle phase ("settle": its extra launches, its length, and the mean launch
time of its first and last windows) beside "warmup".

Launch-bound workloads.  An eager step is a Python call (argument checks, a
ctypes call) of about 10 us, longer than the 256^3 kernel itself, so eager
steps measure the host.  --graph captures the K steps into one HIP graph
and times a replay of it ("launch": "hip_graph" in the JSON line); the
per-launch figure is then a second replay's time per step.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# MI355X bf16 dense MFMA peak: 256 CUs x 4096 flop/clk/CU x 2.4 GHz (published as 2.5 PFLOP/s)
PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12
HBM_PEAK_GBS = 8000.0
# floor of the untimed launches before the timed region (see Settling above)
SETTLE_LAUNCHES = 100
SETTLE_SECONDS = 0.5
SETTLE_WINDOW = 20
CSRC = os.path.join(ROOT, "dense_bf16_gemm_amd", "csrc")


# the headers the benchmarked workloads' kernels are built from, and the host
# code that chooses their tile order and launch
SLAB_SOURCES = ("gemm_kernel.hpp", "gemm_nt_pipe.hpp", "gemm_nt_slab.hpp", "gemm_skinny.hpp", "gemm_small.hpp",
                "mm_api.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in SLAB_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def sclk_path():
    """The driver's GFX clock table (pp_dpm_sclk; its starred line is the
    current clock) when exactly one card exposes one (a single-GPU machine)."""
    paths = glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
    return paths[0] if len(paths) == 1 else None


def read_sclk(path):
    try:
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    m = re.search(r"(\d+)\s*Mhz", line, re.I)
                    return int(m.group(1)) if m else None
    except OSError:
        return None
    return None


def cpu_baseline(w, tensors, target_s: float):
    """The oracle as it stands, on the first R output rows of the workload,
    R grown until one run takes about target_s seconds of loop time."""
    import oracle
    from dense_bf16_gemm_amd import synth

    if w.form == "matmul":
        A = tensors["A"] if "A" in tensors else tensors["At"]
        B = tensors["B"] if "B" in tensors else tensors["Bt"]
        args = dict(A=synth.bits(A), B=synth.bits(B), layout=w.layout, epilogue="none")
    elif w.form == "linear":
        args = dict(A=synth.bits(tensors["x"]), B=synth.bits(tensors["W"]), layout="nt",
                    epilogue=w.epilogue, bias=synth.bits(tensors["bias"]))
    else:
        args = dict(A=synth.bits(tensors["x"]), B=synth.bits(tensors["W_gate"]),
                    B2=synth.bits(tensors["W_up"]), layout="nt", epilogue="swiglu")
    per_row = w.flops / w.M
    rows = 2
    while True:
        _, _, secs = oracle.gemm(rows=(0, rows), timed=True, **args)
        if secs >= target_s * 0.5 or rows >= w.M:
            break
        grow = max(2, int(rows * target_s / max(secs, 1e-3)))
        rows = min(w.M, grow)
    return {
        "value": round(per_row * rows / secs / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "sample": f"first {rows} of {w.M} output rows of {w.name} (all {w.N} columns, full K={w.K}, "
                  f"epilogue included), {secs:.1f} s of loop time",
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--config", default=None, help="tile configuration override (mm_set_config)")
    ap.add_argument("--graph", action="store_true",
                    help="issue the timed steps as one captured HIP graph (for launch-bound "
                         "workloads, whose eager steps measure the host's launch rate)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run three device-to-device copies of BYTES bytes (the reference "
                         "kernel for scaling HBM byte counters) and exit")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: measures one GPU only (asked for {max(args.gpus, world)}); "
              "the GEMM path has no multi-GPU mode", file=sys.stderr)
        return 2

    import torch

    import dense_bf16_gemm_amd as mm
    from dense_bf16_gemm_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 2
    if args.calibrate_copy:
        src = torch.ones(args.calibrate_copy // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"bench: copied {src.numel() * 4} bytes three times", file=sys.stderr)
        return 0
    binding.load()
    if args.config:
        binding.set_config(args.config)
    name = args.workload or synth.HEADLINE
    w = synth.WORKLOADS[name] if name in synth.WORKLOADS else synth.EXTRA_WORKLOADS[name]
    dev = torch.device("cuda:0")
    host = w.make()
    t = {k: v.to(dev) for k, v in host.items()}
    out = torch.empty((w.M, w.N), dtype=torch.float32 if w.out_dtype == "f32" else torch.bfloat16,
                      device=dev)

    if w.form == "matmul":
        Aop = t["A"] if "A" in t else t["At"].t()  # transposed views, read in place
        Bop = t["B"] if "B" in t else t["Bt"].t()
        step = lambda: mm.matmul(Aop, Bop, out.dtype, out=out)  # noqa: E731
    elif w.form == "linear":
        step = lambda: mm.linear(t["x"], t["W"], t["bias"], w.epilogue, out=out)  # noqa: E731
    else:
        step = lambda: mm.ffn_swiglu(t["x"], t["W_gate"], t["W_up"], out=out)  # noqa: E731

    stream = torch.cuda.current_stream()  # the stream every launch goes to
    # --graph: the K steps are captured into a HIP graph before the warm-up
    # (capturing runs nothing, but takes long enough for the clock to drop)
    graph = None
    if args.graph:
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(args.steps):
                step()
        torch.cuda.synchronize()
    settle_t0 = time.perf_counter()
    for _ in range(args.warmup):
        step()
    # settle: windows of launches, each between one event pair, until the
    # floor is reached (none if the warm-up already reached it); one window
    # stays queued behind the one the host waits for, so the GPU never idles
    done, extra, windows, pending = args.warmup, 0, [], []
    while done < SETTLE_LAUNCHES or time.perf_counter() - settle_t0 < SETTLE_SECONDS:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(SETTLE_WINDOW):
            step()
        e1.record(stream)
        pending.append((e0, e1))
        done += SETTLE_WINDOW
        extra += SETTLE_WINDOW
        if len(pending) > 1:
            a, b = pending.pop(0)
            b.synchronize()
            windows.append(a.elapsed_time(b) * 1e3 / SETTLE_WINDOW)
    for a, b in pending:
        b.synchronize()
        windows.append(a.elapsed_time(b) * 1e3 / SETTLE_WINDOW)
    settle = {
        "extra_launches": extra,
        "seconds": round(time.perf_counter() - settle_t0, 3),
        "rule": f">= {SETTLE_LAUNCHES} launches and >= {SETTLE_SECONDS} s of launches before timing",
        "first_window_us": round(windows[0], 1) if windows else None,
        "last_window_us": round(windows[-1], 1) if windows else None,
    }
    # Timed region: the K steps back to back, with one event pair around all
    # of them (events between launches would add their own gaps to it).  With
    # --graph the timed region is one replay of the captured steps.
    torch.cuda.synchronize()
    clock_path = sclk_path()
    t0 = time.perf_counter()
    whole0 = torch.cuda.Event(enable_timing=True)
    whole1 = torch.cuda.Event(enable_timing=True)
    whole0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            step()
    whole1.record(stream)
    # while the GPU works through the timed launches, this thread (no other)
    # samples the clock every millisecond; a step bound by the host's launch
    # rate leaves little to wait for and gets few samples
    sclk = []
    while clock_path and not whole1.query():
        v = read_sclk(clock_path)
        if v is not None:
            sclk.append(v)
        time.sleep(0.001)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = whole0.elapsed_time(whole1)
    # Then the same number of launches again, each between its own events, for
    # the kernel's mean launch duration (the roofline figure).  A graph's
    # launches cannot be bracketed one by one: there the figure is a second
    # replay's mean time per step, gaps between its launches included.
    if graph is not None:
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        graph.replay()
        r1.record(stream)
        torch.cuda.synchronize()
        per_launch = [r0.elapsed_time(r1) / args.steps]
    else:
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        for i in range(args.steps):
            starts[i].record(stream)
            step()
            ends[i].record(stream)
        torch.cuda.synchronize()
        per_launch = [s.elapsed_time(e) for s, e in zip(starts, ends)]  # ms
    ms_per_step = ms_total / args.steps
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    mean_launch = statistics.fmean(per_launch)
    deciles = statistics.quantiles(per_launch, n=10) if len(per_launch) > 1 else per_launch * 9
    achieved = w.flops / (mean_launch * 1e-3) / 1e12

    traffic = traffic_from_profile(name)
    tiles = binding.describe_config(w.form, w.M, w.N, w.K, w.layout)
    cfg = dict(kv.split("=") for kv in tiles.split(","))
    ffn = str(w.form == "ffn").lower()
    # the workspace the step passes ("auto") turns under-filled products into
    # split-K: the slab kernel's split-K instance, then splitk_reduce
    skinny = cfg["KERNEL"] == "gemm_skinny"
    splitk = not skinny and w.form != "ffn" and binding.workspace_size(w.form, w.M, w.N, w.K, w.layout) > 0
    bkn = str(w.layout in ("nn", "tn")).lower()
    amk = str(w.layout in ("tn", "tt")).lower()
    if skinny:
        # at most 16 rows: bound by reading the weight once; with the step's
        # workspace K may be cut into slices (SPLIT=<slices>x<weight rows>)
        kernel = (f"mmk::gemm_skinny<{1 if w.M <= 16 else 2}>" +
                  (" + mmk::skinny_reduce" if "SPLIT" in cfg else ""))
        tiles = f"ROWS=64,SLICES={cfg.get('SPLIT', '1x64').split('x')[0]},KERNEL=gemm_skinny"
    elif splitk:
        # <tile, waves, FFN, split-K, pre-activation output, [K][N] weights,
        # [K][M] activations, bias staged in LDS, ragged K>;
        # SPLIT=<chunks>x<tile width>
        chunks, bn = cfg.get("SPLIT", "0x256").split("x")
        kernel = (f"mmk::gemm_nt_slab<256, {bn}, 2, 2, false, true, false, {bkn}, {amk}, false, false> + "
                  "mmk::splitk_reduce")
        tiles = f"BM=256,BN={bn},WM=2,WN=2,SPLITK={chunks},KERNEL=gemm_nt_slab+splitk_reduce"
    elif cfg["KERNEL"] == "gemm_nt_slab":
        bstage = str(cfg.get("BSTAGE") == "1" and w.form == "linear" and "bias" in w.epilogue
                     and w.layout == "nt").lower()
        ragged = str(w.K % 64 != 0).lower()
        kernel = (f"mmk::gemm_nt_slab<{cfg['BM']}, {cfg['BN']}, {cfg['WM']}, {cfg['WN']}, {ffn}, "
                  f"false, false, {bkn}, {amk}, {bstage}, {ragged}>")
    elif cfg["KERNEL"] == "gemm_small":
        kernel = (f"mmk::gemm_small<{str(w.layout in ('nn', 'nt')).lower()}, "
                  f"{str(w.layout in ('nt', 'tt')).lower()}>")
    elif cfg["KERNEL"] in ("gemm_ws", "gemm_pp"):
        kernel = f"mmk::{cfg['KERNEL']}"
    else:
        kernel = f"mmk::{cfg['KERNEL']}<{cfg['BM']}, {cfg['BN']}, {cfg['WM']}, {cfg['WN']}, {ffn}>"
    result = {
        "metric": "TFLOP/s and % of bf16 MFMA peak, 8192^3 linear+bias+GELU, 1 GPU"
        if name == synth.HEADLINE else f"TFLOP/s, {name}, 1 GPU",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "launch": "hip_graph" if graph is not None else "stream",
        "settle": settle,
        "sclk_mhz": ({"median": statistics.median(sclk), "min": min(sclk), "max": max(sclk),
                      "samples": len(sclk),
                      "source": "pp_dpm_sclk (current level) while the timed launches ran"}
                     if sclk else None),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": name,
            "form": w.form,
            "M": w.M, "N": w.N, "K": w.K,
            "layout": w.layout,
            "epilogue": w.epilogue,
            "out_dtype": w.out_dtype,
            "tiles": tiles,
            "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
            "device": torch.cuda.get_device_name(dev),
            "arch": getattr(torch.cuda.get_device_properties(dev), "gcnArchName", None),
            "compute_units": torch.cuda.get_device_properties(dev).multi_processor_count,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_BF16_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": kernel,
            "launch_ms_mean": round(mean_launch, 5),
            "launch_ms_median": round(statistics.median(per_launch), 5),
            "launch_ms_min": round(min(per_launch), 5),
            "launch_ms_p10": round(deciles[0], 5),
            "launch_ms_p90": round(deciles[-1], 5),
        },
        "cpu_baseline": None,
    }
    if skinny:
        # the weight read once bounds it: algorithmic bytes per launch over
        # the mean launch time, against the 8 TB/s of HBM
        gbs = w.algorithmic_bytes / (mean_launch * 1e-3) / 1e9
        result["roofline"].update({"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                                   "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                                   "bytes_per_launch": w.algorithmic_bytes})
    print(f"bench: {name}: {ms_per_step * 1e3:.1f} us/step, {value:.1f} TFLOP/s "
          f"({100 * value / PEAK_BF16_TFLOPS:.1f}% of peak), wall {wall:.3f} s", file=sys.stderr,
          flush=True)
    if not args.no_cpu_baseline:
        del t
        result["cpu_baseline"] = cpu_baseline(w, host, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
