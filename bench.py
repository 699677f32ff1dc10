#!/usr/bin/env python3
"""Benchmark of the channels-last conv forward hot path on one MI355X.

Workload (default): the fp32 conv2d the Winograd-tiling MLX PR ("Bound
winograd conv2d working set by tiling the batch", Testing) reports on --
N=40 x 512x512, C=192 -> O=96, 3x3, stride 1, pad 1, x ~ U[-1,1],
w ~ N(0, 1/(9C)), seeded and synthetic.  One step is one full forward call
(plan selection, then every kernel of the selected algorithm: for this
workload the Winograd filter transform, input transform, 64 tile-position
GEMMs and output transform, over the batch tiles the byte budget allows).

Metric: direct-equivalent TFLOP/s = 2*N*OH*OW*O*C*KH*KW / time per step, with
inputs resident in HBM.  Per-kernel durations come from hipEvents the library
records on the launch stream between kernels during the timed steps; the
dominant kernel is reported against its roofline (algorithmic flops or bytes
per launch / average launch time).  The CPU baseline times the fp64 oracle on
a bounded sample of output pixels of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch N]
                       [--ws-limit BYTES] [--tile-batch T] [--no-cpu-baseline]
Prints one JSON line on stdout; progress goes to stderr.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {  # MI355X published peaks
    "hbm_gbs": 8000.0,
    "mfma_tflops": {"f32": 157.3, "f16": 2500.0, "bf16": 2500.0},
}
PAGE_BASELINE_TFLOPS = 11.2  # the page's ~310 ms Winograd time on this workload, direct-equivalent (M2 Max)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--batch", type=int, default=40)
    ap.add_argument("--ws-limit", type=int, default=None)
    ap.add_argument("--tile-batch", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (small fp32, budgets, half sweep, ResNet-50 stack, video 3D)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calib-copy", type=int, default=0,
                    help="also run one plain device copy of this many bytes (fp32 -> fp32) before the "
                         "timed work, as the known-size reference for HBM traffic counters")
    ap.add_argument("--traffic-from", nargs=2, default=None, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="parse two rocprofv3 --pmc counter CSVs (FETCH_SIZE, WRITE_SIZE) of a run made "
                         "with --calib-copy, write profiles/traffic.json, print it and exit")
    ap.add_argument("--suite", default=None,
                    help="instead of the headline line, time other workloads: "
                         "comma list of small,wide,sweep,wino_half,resnet,video,video_auto,video_gemm,big_gemm,conv1d,"
                         "vendor_gemm "
                         "or 'all' "
                         "(one JSON line each)")
    return ap.parse_args()


# The sources the headline workload's kernels (the fp32 Winograd transforms and
# the resident Winograd GEMM) are compiled from, headers included (and the
# public header include/cnhwc.h, which they include too).
HEADLINE_SOURCES = ("winograd.hip", "wino_gemm.hip", "wino_f63_api.hpp", "wino_mask.hpp", "device_common.hpp",
                    "winograd_f63.h")


def _code_only(text):
    """Source text without comments and with whitespace runs collapsed."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def csrc_hash():
    """Hash of the headline kernels' sources, comments and layout aside
    (decides whether stored traffic counters still apply: a change to the code
    of any of them voids the counters)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "convolution_nhwc_conv2d_amd", "csrc")
    for f in HEADLINE_SOURCES:
        h.update(f.encode())
        h.update(_code_only(open(os.path.join(d, f)).read()).encode())
    h.update(_code_only(open(os.path.join(ROOT, "include", "cnhwc.h")).read()).encode())
    return h.hexdigest()[:16]


def kernel_work(kind, plan, case, es):
    """Algorithmic work of one launch of a kernel kind for this plan:
    (bound, amount, unit).  Flops for GEMM stages, HBM bytes for transforms."""
    n, h, w, c, o = plan.tile_batch, case.h, case.w, case.c, case.o
    cs = (c + 7) // 8 * 8
    rows = n * plan.tiles_per_image
    if kind == "wino_gemm":
        return "mfma", 2.0 * 64 * rows * c * o, "flop"
    if kind == "wino_input":
        return "hbm", float(n * h * w * c * es + 64 * rows * cs * 4), "byte"
    if kind == "wino_output":
        return "hbm", float(64 * rows * o * 4 + n * plan.out_h * plan.out_w * o * es), "byte"
    if kind == "wino_filter":
        return "hbm", float(o * 9 * c * es + 64 * o * cs * 4), "byte"
    if kind == "implicit_gemm":
        m = case.n * plan.out_h * plan.out_w
        return "mfma", 2.0 * m * o * case.kh * case.kw * c, "flop"
    return None, None, None


def load_traffic(workload_key, kind):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        data = json.load(open(path))
    except ValueError:
        return None
    ent = data.get(workload_key, {}).get(kind)
    if not ent or ent.get("csrc_hash") != csrc_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(case, seconds):
    """Time the fp64 oracle on a seeded sample of output pixels (all O channels)."""
    import numpy as np
    import oracle
    import conv_workloads as cw
    threads = len(os.sched_getaffinity(0))
    w = case.weight().numpy()
    per = case.h * case.w  # output pixels per batch element (3x3, s1, p1: OH=H, OW=W)
    kw = case.conv_kwargs()
    x1 = case.input([0]).numpy()
    calib = cw.sample_rows(per, 4096, 11)
    t0 = time.perf_counter()
    oracle.conv(x1, w, **kw, rows=calib, threads=threads)
    rate = calib.size / (time.perf_counter() - t0)
    # the sample: seeded output pixels spread over the first `elems` batch elements
    count = int(max(4096, rate * seconds))
    elems = min(case.n, -(-count // per))
    count = min(count, elems * per)
    xs = case.input(list(range(elems))).numpy()
    rows = cw.sample_rows(elems * per, count, 12)
    t0 = time.perf_counter()
    yr, den = oracle.conv(xs, w, **kw, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    flops = 2.0 * count * case.o * case.kh * case.kw * case.c
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{count} seeded output pixels (x {case.o} channels) of batch elements 0..{elems - 1}, "
                      f"fp64 direct correlation, {dt:.2f} s wall; CPU {cpu}",
            "seconds": dt, "outputs_per_s": count * case.o / dt,
            # extrapolated, not measured: the sample's rate over all case.n * OH * OW pixels
            "extrapolated_full_s": dt * (case.n * per) / count,
            # the sample's fp64 results, for the parity check of the GPU output (not printed)
            "_rows": rows, "_y": yr, "_den": den}


def traffic_from(fetch_csv, write_csv, calib_bytes, workload_key):
    """Per-launch HBM bytes of each kernel kind from two rocprofv3 --pmc runs,
    each counter scaled so that the plain copy of `calib_bytes` reads (writes)
    exactly `calib_bytes`.  Kernel kinds are recognised by kernel name."""
    import csv
    kinds = {"wino_input_kernel": "wino_input", "wino_output_kernel": "wino_output",
             "wino_filter_kernel": "wino_filter", "wino_gemm_resident_kernel": "wino_gemm",
             "gemm_kernel": "gemm", "unfold_": "unfold"}

    def load(path, counter):
        per = {}
        for row in csv.DictReader(open(path)):
            if row.get("Counter_Name") != counter:
                continue
            name = row.get("Kernel_Name", "")
            kind = next((v for k, v in kinds.items() if k in name), None)
            if kind is None and ("copy" in name.lower() or "elementwise" in name.lower()):
                kind = "copy"
            if kind is None:
                continue
            per.setdefault(kind, []).append(float(row["Counter_Value"]))
        return per

    f = load(fetch_csv, "FETCH_SIZE")
    w = load(write_csv, "WRITE_SIZE")
    kib = calib_bytes / 1024.0
    ffac = kib / max(f["copy"]) if f.get("copy") else None
    wfac = kib / max(w["copy"]) if w.get("copy") else None
    out = {"calib_copy_bytes": calib_bytes, "fetch_scale": ffac, "write_scale": wfac,
           "csrc_hash": csrc_hash(), "kernels": {}}
    for kind in set(f) | set(w):
        if kind == "copy":
            continue
        fk = sum(f.get(kind, [0])) / max(1, len(f.get(kind, [0])))
        wk = sum(w.get(kind, [0])) / max(1, len(w.get(kind, [0])))
        out["kernels"][kind] = {"fetch_kib_raw": fk, "write_kib_raw": wk,
                                "bytes_per_launch": (fk * (ffac or 1) + wk * (wfac or 1)) * 1024.0,
                                "csrc_hash": csrc_hash()}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[workload_key] = out["kernels"]
    data[workload_key + ":calibration"] = {k: v for k, v in out.items() if k != "kernels"}
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    return out


# Bytes written between repetitions of the cold timing variant (twice the
# 256 MB Infinity Cache), and the GPU spin (clock cycles, about 50 us) that
# spaces the warm variant.
COLD_BYTES = 512 << 20
SPIN_CYCLES = 100_000


def _time_call(fn, reps=15, warmup=3, flush=None):
    """Median ms per call of fn() on the current stream (torch events around
    each call), so that a one-off stall of the machine does not move the
    figure; the minimum is in _time_call.last_min.  flush, if given, runs
    before each timed call, outside its events (the cold variant)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        if flush is not None:
            flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    _time_call.last_min = t[0]
    return t[len(t) // 2]


def _kernel_split(fn, reps=3):
    """Per-kernel-kind average ms of fn(timer) over reps calls."""
    import convolution_nhwc_conv2d_amd as cn
    import torch
    t = cn.KernelTimer()
    for _ in range(reps):
        fn(t)
    torch.cuda.synchronize()
    agg = {}
    for kind, ms in t.durations():
        agg[kind] = agg.get(kind, 0.0) + ms / reps
    t.close()
    return agg


def run_suite(names):
    """Time the other workloads of the pages; one JSON line per measurement."""
    import torch
    import conv_workloads as cw
    import convolution_nhwc_conv2d_amd as cn
    dev = torch.device("cuda:0")

    def emit(d):
        print(json.dumps(d), flush=True)

    flush_buf = torch.empty(COLD_BYTES, dtype=torch.uint8, device=dev)

    def measure(case, algo="auto", inner=None, **kw):
        x = case.input().to(dev)
        w = case.weight().to(dev)
        fn = cn.conv2d if case.nd == 2 else cn.conv3d
        extra = dict(kw)
        if inner:
            extra["inner_algo"] = inner
        y = fn(x, w, **case.conv_kwargs(), algo=algo, **extra)
        plan = (cn.plan2d if case.nd == 2 else cn.plan3d)(tuple(x.shape), tuple(w.shape), **case.conv_kwargs(),
                                                          dtype=x.dtype, algo=algo, **extra)
        ws = torch.empty(max(1, plan.workspace_bytes), dtype=torch.uint8, device=dev)
        call = lambda timer=None: fn(x, w, **case.conv_kwargs(), plan=plan, out=y, workspace=ws, timer=timer)
        ms = _time_call(call)
        ms_min = _time_call.last_min
        split = _kernel_split(call)
        flops = cn.direct_flops(tuple(x.shape), tuple(w.shape), plan)
        r = {"workload": case.name, "dtype": case.dtype, "algo": plan.algo_name,
             "inner_algo": plan.inner_algo_name, "ms": ms, "ms_min": ms_min, "tflops": flops / ms / 1e9,
             "kernels_ms": split, "flops": flops}
        # Working sets that fit the 256 MB Infinity Cache stay warm across
        # repeated calls.  Two spaced variants put GPU work before each call,
        # so the host's launch overhead is hidden in both and only the cache
        # state differs: a spin that touches no memory (warm) and a 512 MB
        # write (cold).  "ms" stays the back-to-back figure.
        working = sum(t.numel() * t.element_size() for t in (x, w, y, ws))
        if working < COLD_BYTES // 2:
            r["ms_warm_spaced"] = _time_call(call, flush=lambda: torch.cuda._sleep(SPIN_CYCLES))
            r["ms_cold"] = _time_call(call, flush=lambda: flush_buf.fill_(1))
            r["tflops_cold"] = flops / r["ms_cold"] / 1e9
        return r

    if "small" in names:
        for algo in ("winograd", "implicit_gemm", "unfold_gemm", "auto"):
            r = measure(cw.small_fp32(), algo)
            r["suite"] = "small_fp32"
            emit(r)
    if "wide" in names:
        for n in (8, 32, 40, 64):
            case = cw.wide_fp32(n)
            for wl in (None, 40_200_000_000, 512 * 10**6):
                kw = {} if wl is None else {"ws_limit": wl}
                r = measure(case, **kw)
                r.update(suite="wide_fp32", ws_limit=wl)
                emit(r)
    if "sweep" in names:
        for dt in ("f16", "bf16"):
            for c_out in (128, 256, 512, 1024, 2048, 4096):
                for n in (1, 4, 16, 64):
                    case = cw.cout_axis(dt, c_out, n)
                    res = {a: measure(case, a) for a in ("implicit_gemm", "unfold_gemm")}
                    emit({"suite": "half_cout_axis", "dtype": dt, "c_out": c_out, "m": n * 1024,
                          "implicit_ms": res["implicit_gemm"]["ms"], "unfold_ms": res["unfold_gemm"]["ms"],
                          "implicit_tflops": res["implicit_gemm"]["tflops"],
                          "unfold_tflops": res["unfold_gemm"]["tflops"],
                          "unfold_over_implicit": res["implicit_gemm"]["ms"] / res["unfold_gemm"]["ms"]})
            for c_in in (128, 256, 512, 1024):
                case = cw.cout_axis(dt, 1024, 16, c_in)
                res = {a: measure(case, a) for a in ("implicit_gemm", "unfold_gemm")}
                emit({"suite": "half_k_axis", "dtype": dt, "k": 9 * c_in, "c_out": 1024, "m": 16384,
                      "implicit_tflops": res["implicit_gemm"]["tflops"],
                      "unfold_tflops": res["unfold_gemm"]["tflops"],
                      "unfold_over_implicit": res["implicit_gemm"]["ms"] / res["unfold_gemm"]["ms"]})
    if "resnet" in names:
        for batch in (1, 8):
            stages = {}
            for case, mult, stage in cw.resnet50_layers(batch):
                r = measure(case)
                s_ = stages.setdefault(stage, {"ms": 0.0, "ms_warm_spaced": 0.0, "ms_cold": 0.0, "flops": 0.0})
                s_["ms"] += r["ms"] * mult
                s_["ms_warm_spaced"] += r.get("ms_warm_spaced", r["ms"]) * mult
                s_["ms_cold"] += r.get("ms_cold", r["ms"]) * mult
                s_["flops"] += r["flops"] * mult
                emit({"suite": "resnet50_layer", "batch": batch, "layer": case.name, "mult": mult,
                      "algo": r["algo"], "ms": r["ms"], "ms_warm_spaced": r.get("ms_warm_spaced"),
                      "ms_cold": r.get("ms_cold"), "tflops": r["tflops"],
                      "kernels_ms": r["kernels_ms"]})
            tot_ms = sum(v["ms"] for v in stages.values())
            tot_cold = sum(v["ms_cold"] for v in stages.values())
            tot_spaced = sum(v["ms_warm_spaced"] for v in stages.values())
            tot_fl = sum(v["flops"] for v in stages.values())
            emit({"suite": "resnet50_stack", "batch": batch, "dtype": "f16", "total_ms": tot_ms,
                  "total_ms_warm_spaced": tot_spaced, "total_ms_cold": tot_cold, "tflops": tot_fl / tot_ms / 1e9,
                  "stages_ms": {k: v["ms"] for k, v in stages.items()}})
            # the same 53 convs captured once into a HIP graph and replayed: the
            # GPU time of the stack without the per-call host overhead
            calls, flops = [], 0.0
            for case, mult, stage in cw.resnet50_layers(batch):
                x = case.input().to(dev)
                w = case.weight().to(dev)
                plan = cn.plan2d(tuple(x.shape), tuple(w.shape), **case.conv_kwargs(), dtype=x.dtype)
                ws = torch.empty(max(1, plan.workspace_bytes), dtype=torch.uint8, device=dev)
                y = cn.conv2d(x, w, **case.conv_kwargs(), plan=plan, workspace=ws)
                for _ in range(mult):
                    calls.append((x, w, case, plan, ws, y))
                    flops += cn.direct_flops(tuple(x.shape), tuple(w.shape), plan)
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                for x, w, case, plan, ws, y in calls:
                    cn.conv2d(x, w, **case.conv_kwargs(), plan=plan, workspace=ws, out=y)
                torch.cuda.synchronize()
                with torch.cuda.graph(graph, stream=side):
                    for x, w, case, plan, ws, y in calls:
                        cn.conv2d(x, w, **case.conv_kwargs(), plan=plan, workspace=ws, out=y)
            ms = _time_call(graph.replay)
            emit({"suite": "resnet50_stack_graph", "batch": batch, "dtype": "f16", "convs": len(calls),
                  "total_ms": ms, "total_ms_min": _time_call.last_min, "tflops": flops / ms / 1e9})
            del calls, graph
    if "video" in names:
        for shape in cw.VIDEO3D_SHAPES:
            case = cw.video3d(*shape)
            # AUTO (half-precision Winograd, taps summed in its GEMMs), the native
            # 3D implicit GEMM, and the per-tap decomposition with each inner path
            for algo, inner in (("auto", None), ("implicit_gemm", None), ("auto", "implicit_gemm"),
                                ("auto", "unfold_gemm")):
                r = measure(case, algo, inner=inner)
                r["suite"] = "video3d"
                emit(r)
    if "video_gemm" in names:
        # the GEMM-only paths on the video shapes, for profiles: the native 3D
        # implicit GEMM and the per-tap decomposition with each inner path
        for shape in cw.VIDEO3D_SHAPES:
            case = cw.video3d(*shape)
            for algo, inner in (("implicit_gemm", None), ("small_kd", "implicit_gemm"), ("small_kd", "unfold_gemm")):
                r = measure(case, algo, inner=inner)
                r["suite"] = "video3d_gemm"
                emit(r)
    if "video_auto" in names:
        # the AUTO path alone (half-precision Winograd) on the video shapes, for profiles
        for shape in cw.VIDEO3D_SHAPES:
            r = measure(cw.video3d(*shape))
            r["suite"] = "video3d_auto"
            emit(r)
    if "big_gemm" in names:
        # the largest half-precision GEMM stages alone, for counter profiles:
        # the C_out 4096 implicit GEMM (65536 x 4096 x 2304) in f16 and bf16,
        # the K-axis one (16384 x 1024 x 9216), the native 3D video GEMM
        # (973440 x 512 x 13824) and the video conv on AUTO (half-precision
        # Winograd, taps summed in its GEMMs)
        for dt in ("f16", "bf16"):
            r = measure(cw.cout_axis(dt, 4096, 64), "implicit_gemm")
            r["suite"] = "big_gemm"
            emit(r)
        r = measure(cw.cout_axis("f16", 1024, 16, 1024), "implicit_gemm")
        r["suite"] = "big_gemm"
        emit(r)
        for algo in ("implicit_gemm", "auto"):
            r = measure(cw.video3d(41, 120, 208, 512, 512), algo)
            r["suite"] = "big_gemm"
            emit(r)
    if "wino_half" in names:
        # half-precision Winograd F(4x4,3x3) against the implicit GEMM around
        # AUTO's crossover (3x3 s1 p1 on 32x32)
        for dt in ("f16", "bf16"):
            for c, o in ((256, 256), (256, 512), (512, 256), (512, 512), (1024, 512), (1024, 1024), (2048, 512)):
                for n in (16, 64):
                    case = cw.cout_axis(dt, o, n, c)
                    res = {a: measure(case, a) for a in ("implicit_gemm", "winograd_half")}
                    auto = cn.plan2d(case.x_shape(), case.w_shape(), **case.conv_kwargs(),
                                     dtype=cw.DTYPES[dt]).algo_name
                    emit({"suite": "wino_half", "dtype": dt, "c_in": c, "c_out": o, "m": n * 1024, "auto": auto,
                          "implicit_ms": res["implicit_gemm"]["ms"], "wino_half_ms": res["winograd_half"]["ms"],
                          "implicit_tflops": res["implicit_gemm"]["tflops"],
                          "wino_half_tflops": res["winograd_half"]["tflops"],
                          "wino_half_kernels_ms": res["winograd_half"]["kernels_ms"],
                          "speedup": res["implicit_gemm"]["ms"] / res["winograd_half"]["ms"]})
    if "conv1d" in names:
        # Whisper-large-shaped encoder convs (128 log-mel bins -> 1280, k3 p1;
        # 1280 -> 1280, k3 s2 p1) over 3000 frames, through the 2D path (H = 1)
        for batch in (1, 8):
            for c, o, s in ((128, 1280, 1), (1280, 1280, 2)):
                case = cw.ConvCase(f"conv1d_f16_b{batch}_{c}to{o}_k3s{s}", batch, 1, 3000, c, o, 1, 3, (1, s),
                                   (0, 1), (1, 1), "f16", "normal", "normal", None, 6, c + s)
                r = measure(case)
                r["suite"] = "conv1d"
                emit(r)
    if "vendor_gemm" in names:
        # Reference point for the half-precision GEMM stages, not part of the
        # path: the vendor GEMM (torch.matmul) on dense operands of the same
        # M x N x K as the large implicit GEMMs (the C_out and K axes of the
        # sweep, the largest video conv's per-tap GEMM) and a square 8192^3.
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        for dt in (torch.float16, torch.bfloat16):
            for m, n, k in ((16384, 1024, 9216), (65536, 4096, 2304), (16384, 1024, 2304), (65536, 256, 2304),
                            (973440, 512, 4608), (8192, 8192, 8192)):
                a = torch.randn((m, k), device=dev, dtype=dt, generator=gen)
                b = torch.randn((k, n), device=dev, dtype=dt, generator=gen)
                c = torch.empty((m, n), device=dev, dtype=dt)
                ms = _time_call(lambda timer=None: torch.matmul(a, b, out=c))
                emit({"suite": "vendor_gemm", "dtype": str(dt).replace("torch.", ""), "m": m, "n": n, "k": k,
                      "ms": ms, "tflops": 2.0 * m * n * k / ms / 1e9})
                del a, b, c


def _gemm_work(kind, plan, case):
    """Algorithmic flops of all launches of a GEMM kernel kind in one call (None
    if the kind is not a GEMM stage)."""
    k3 = case.kd * case.kh * case.kw * case.c
    m = case.n * plan.out_d * plan.out_h * plan.out_w
    if kind in ("implicit_gemm", "unfold_gemm"):
        return 2.0 * m * case.o * k3
    if kind == "wino_gemm":
        if plan.algo_name == "winograd_half":
            cs = -(-case.c // 32) * 32
            return 2.0 * 36 * case.n * plan.out_d * plan.tiles_per_image * case.o * case.kd * cs
        return 2.0 * 64 * case.n * plan.tiles_per_image * case.c * case.o
    return None


def _gemm_peak(plan, dtype):
    """MFMA peak of the GEMM stages' operand type: the half Winograd path runs
    fp16 operands for bf16 inputs too; the fp32 Winograd path fp32 operands."""
    if plan.algo_name == "winograd" or plan.inner_algo_name == "winograd" or dtype == "f32":
        return PEAK["mfma_tflops"]["f32"]
    return PEAK["mfma_tflops"]["f16"]


def _oracle_sample(case, x, w, y, count, seed, threads):
    """The GPU output against the fp64 oracle on `count` seeded output rows
    (all O channels each)."""
    import numpy as np
    import torch
    import conv_workloads as cw
    import oracle
    o = y.shape[-1]
    total = y.numel() // o
    rows = cw.sample_rows(total, count, seed)
    yr, den = oracle.conv(x.float().numpy(), w.float().numpy(), **case.conv_kwargs(), rows=rows, threads=threads)
    idx = torch.as_tensor(rows, device=y.device, dtype=torch.long)
    yg = y.reshape(-1, o).index_select(0, idx).double().cpu().numpy()
    tol = 2e-5 if case.dtype == "f32" else 1e-2
    err = np.abs(yg - yr)
    zero = den == 0
    rel = err[~zero] / den[~zero]
    ok = bool(np.all(yg[zero] == 0) and np.all(err[~zero] <= tol * den[~zero]))
    return {"outputs": int(yr.size), "max_err_over_sum_abs": float(rel.max()) if rel.size else 0.0,
            "tol": tol, "within_tol": ok}


def run_configs(dev, head):
    """The other four workloads (and the headline's budget variants), each with
    median and min ms over 15 back-to-back calls, the direct-equivalent rate,
    the dominant kernel against its roofline and an oracle check on a seeded
    sample of output rows."""
    import torch
    import conv_workloads as cw
    import convolution_nhwc_conv2d_amd as cn
    threads = len(os.sched_getaffinity(0))
    out = {}

    def timed(case, x, w, algo="auto", plan=None, y=None, **kw):
        fn = cn.conv2d if case.nd == 2 else cn.conv3d
        if plan is None:
            plan = (cn.plan2d if case.nd == 2 else cn.plan3d)(tuple(x.shape), tuple(w.shape), **case.conv_kwargs(),
                                                              dtype=x.dtype, algo=algo, **kw)
        oshape = (x.shape[0],) + ((plan.out_d,) if case.nd == 3 else ()) + (plan.out_h, plan.out_w, case.o)
        y = torch.empty(oshape, dtype=x.dtype, device=dev) if y is None else y
        ws = torch.empty(max(1, plan.workspace_bytes), dtype=torch.uint8, device=dev)
        call = lambda timer=None: fn(x, w, **case.conv_kwargs(), plan=plan, out=y, workspace=ws, timer=timer)
        ms = _time_call(call)
        ms_min = _time_call.last_min
        split = _kernel_split(call)
        flops = cn.direct_flops(tuple(x.shape), tuple(w.shape), plan)
        gemms = [k for k in split if _gemm_work(k, plan, case) is not None]
        dom = max(gemms, key=split.get) if gemms else None
        work = _gemm_work(dom, plan, case) if dom else None
        ent = {"algo": plan.algo_name, "ms_median": ms, "ms_min": ms_min, "tflops": flops / ms / 1e9,
               "kernels_ms": split}
        if work is not None:
            peak = _gemm_peak(plan, case.dtype)
            ach = work / (split[dom] / 1e3) / 1e12
            ent["dominant"] = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                               "frac": ach / peak}
        del ws
        return ent, y, plan

    # small fp32 (latency-bound: microseconds)
    case = cw.small_fp32()
    x, w = case.input(), case.weight()
    xg, wg = x.to(dev), w.to(dev)
    ents = []
    for algo in ("winograd", "implicit_gemm", "auto"):
        e, y, _ = timed(case, xg, wg, algo)
        e = {"algo": e["algo"], "forced": algo != "auto", "us_median": e["ms_median"] * 1e3,
             "us_min": e["ms_min"] * 1e3, "kernels_ms": e["kernels_ms"],
             "oracle_check": _oracle_sample(case, x, w, y, 256, 21, threads)}
        ents.append(e)
    out["small_fp32"] = {"workload": "conv2d fp32 NHWC N=1, 16x16, 32->32, 3x3, stride 1, pad 1",
                         "bound": "latency", "entries": ents}
    log("[bench] configs: small fp32 done")

    # the headline conv under the injected budgets: 40.2e9 (batch tiles) and 512 MB (fallback)
    hcase, hx, hw, hy = head
    ents = []
    for wl in (40_200_000_000, 512 * 10**6):
        e, y, plan = timed(hcase, hx, hw, ws_limit=wl, y=hy)
        e.update(ws_limit_bytes=wl, tile_batch=plan.tile_batch, n_tiles=plan.n_tiles,
                 oracle_check=_oracle_sample(hcase, hcase.input([0]), hcase.weight(), y[:1], 256, 22, threads))
        ents.append(e)
    out["wide_fp32_budgets"] = {"workload": f"conv2d fp32 NHWC N={hcase.n}, 512x512, 192->96, 3x3, s1, p1",
                                "entries": ents}
    log("[bench] configs: wide fp32 budgets done")

    # half-precision sweep: the widest C_out at the largest M, both dtypes, and an unaligned C_in
    ents = []
    for dt, c_out, n, c_in in (("f16", 4096, 64, 256), ("bf16", 4096, 64, 256), ("f16", 1024, 16, 1000)):
        case = cw.cout_axis(dt, c_out, n, c_in)
        x, w = case.input(), case.weight()
        xg, wg = x.to(dev), w.to(dev)
        for algo in ("auto", "unfold_gemm"):
            e, y, _ = timed(case, xg, wg, algo)
            e.update(workload=f"{dt} 32x32 {c_in}->{c_out} 3x3 s1 p1, M={n * 1024}, K={9 * c_in}",
                     oracle_check=_oracle_sample(case, x, w, y, 256, 23, threads))
            ents.append(e)
        del xg, wg
    out["half_sweep"] = {"workload": "conv2d fp16/bf16 C_out axis and unaligned C_in", "entries": ents}
    log("[bench] configs: half sweep done")

    # the ResNet-50 conv stack: each conv eager, and the whole stack replayed as one HIP graph
    ents = []
    for batch in (1, 8):
        calls, flops, eager_ms, gemm_flops, gemm_ms, worst = [], 0.0, 0.0, 0.0, 0.0, 0.0
        ok = True
        for case, mult, stage in cw.resnet50_layers(batch):
            x, w = case.input(), case.weight()
            xg, wg = x.to(dev), w.to(dev)
            e, y, plan = timed(case, xg, wg)
            chk = _oracle_sample(case, x, w, y, 64, 24, threads)
            ok = ok and chk["within_tol"]
            worst = max(worst, chk["max_err_over_sum_abs"])
            eager_ms += e["ms_median"] * mult
            for kind, kms in e["kernels_ms"].items():
                g = _gemm_work(kind, plan, case)
                if g is not None:
                    gemm_flops += g * mult
                    gemm_ms += kms * mult
            ws = torch.empty(max(1, plan.workspace_bytes), dtype=torch.uint8, device=dev)
            for _ in range(mult):
                calls.append((xg, wg, case, plan, ws, y))
                flops += cn.direct_flops(tuple(xg.shape), tuple(wg.shape), plan)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            for x_, w_, case, plan, ws, y in calls:
                cn.conv2d(x_, w_, **case.conv_kwargs(), plan=plan, workspace=ws, out=y)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=side):
                for x_, w_, case, plan, ws, y in calls:
                    cn.conv2d(x_, w_, **case.conv_kwargs(), plan=plan, workspace=ws, out=y)
        gms = _time_call(graph.replay)
        ents.append({"batch": batch, "convs": len(calls), "eager_ms_sum_of_medians": eager_ms,
                     "graph_ms_median": gms, "graph_ms_min": _time_call.last_min, "tflops_graph": flops / gms / 1e9,
                     "bound": "latency",
                     "gemm_kernels": {"achieved": gemm_flops / (gemm_ms / 1e3) / 1e12,
                                      "peak": PEAK["mfma_tflops"]["f16"], "unit": "TFLOP/s",
                                      "frac": gemm_flops / (gemm_ms / 1e3) / 1e12 / PEAK["mfma_tflops"]["f16"]},
                     "oracle_check": {"outputs": "64 seeded rows x O of each of the 23 convs",
                                      "max_err_over_sum_abs": worst, "tol": 1e-2, "within_tol": ok}})
        del calls, graph
    out["resnet50_fp16"] = {"workload": "ResNet-50 v1.5 conv stack fp16, 224x224x3, 53 convs", "entries": ents}
    log("[bench] configs: resnet50 stack done")

    # video conv3d bf16 on AUTO (half-precision Winograd with the depth taps in its GEMMs)
    ents = []
    for shape in cw.VIDEO3D_SHAPES:
        case = cw.video3d(*shape)
        x, w = case.input(), case.weight()
        xg, wg = x.to(dev), w.to(dev)
        e, y, _ = timed(case, xg, wg)
        e.update(workload=f"bf16 {shape[0]}x{shape[1]}x{shape[2]} {shape[3]}->{shape[4]} 3x3x3 pad (0,1,1)",
                 oracle_check=_oracle_sample(case, x, w, y, 256, 25, threads))
        ents.append(e)
        del xg, wg, y, x
    out["video3d_bf16"] = {"workload": "conv3d bf16 NDHWC N=1, 3x3x3, stride 1, pad (0,1,1)", "entries": ents}
    log("[bench] configs: video 3D done")
    return out


def main():
    args = parse()
    if args.traffic_from:
        key = f"fp32_{args.batch}x512x512_192to96"
        print(json.dumps(traffic_from(args.traffic_from[0], args.traffic_from[1], args.calib_copy, key), indent=1))
        return
    if args.suite:
        names = ({"small", "wide", "sweep", "wino_half", "resnet", "video", "conv1d"} if args.suite == "all"
                 else set(args.suite.split(",")))
        run_suite(names)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(each GPU would run the same plan on its own share of the batch).", file=sys.stderr)
        sys.exit(2)

    import torch
    import conv_workloads as cw
    import convolution_nhwc_conv2d_amd as cn

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    case = cw.wide_fp32(args.batch)
    log(f"[bench] generating {case.name} inputs")
    t0 = time.perf_counter()
    w = case.weight().to(dev)
    x = torch.empty(case.x_shape(), dtype=torch.float32, device=dev)
    for i in range(case.n):
        x[i].copy_(case.element(i))
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")

    ws_limit = args.ws_limit if args.ws_limit is not None else cn.default_ws_limit(dev)
    plan = cn.plan2d(tuple(x.shape), tuple(w.shape), 1, 1, 1, torch.float32, ws_limit=ws_limit,
                     tile_batch=args.tile_batch)
    log(f"[bench] plan {plan}")
    out = torch.empty((case.n, plan.out_h, plan.out_w, case.o), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, plan.workspace_bytes), dtype=torch.uint8, device=dev)

    def step(timer=None):
        cn.conv2d(x, w, 1, 1, 1, plan=plan, out=out, workspace=ws, timer=timer)

    if args.calib_copy:
        src = torch.ones(args.calib_copy // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"[bench] calibration copy of {args.calib_copy} bytes done")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} done; timing {args.steps} steps")
    timer = cn.KernelTimer()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(timer)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt * 1e3 / args.steps
    flops = cn.direct_flops(tuple(x.shape), tuple(w.shape), plan)
    value = flops / (ms / 1e3) / 1e12
    log(f"[bench] {ms:.3f} ms/step, {value:.2f} TFLOP/s direct-equivalent")

    per_kind = {}
    durations = timer.durations()
    spans = sorted(timer.call_ms)
    for kind, kms in durations:
        e = per_kind.setdefault(kind, [0, 0.0])
        e[0] += 1
        e[1] += kms
    timer.close()
    stages = {}
    for kind, (cnt, tot) in per_kind.items():
        bound, work, unit = kernel_work(kind, plan, case, 4)
        avg = tot / cnt
        ent = {"launches": cnt, "avg_ms": avg, "share": tot / (ms * args.steps)}
        if bound == "mfma":
            ent.update(bound="mfma", achieved=work / (avg / 1e3) / 1e12, peak=PEAK["mfma_tflops"]["f32"],
                       unit="TFLOP/s", work_per_launch=work)
            ent["frac"] = ent["achieved"] / ent["peak"]
        elif bound == "hbm":
            ent.update(bound="hbm", achieved=work / (avg / 1e3) / 1e9, peak=PEAK["hbm_gbs"], unit="GB/s",
                       work_per_launch=work)
            ent["frac"] = ent["achieved"] / ent["peak"]
        stages[kind] = ent
    dom = max(stages, key=lambda k: stages[k]["avg_ms"] * stages[k]["launches"])
    d = stages[dom]
    traffic = load_traffic(f"fp32_{case.n}x512x512_192to96", dom)
    roofline = {"bound": d.get("bound"), "achieved": d.get("achieved"), "peak": d.get("peak"),
                "unit": d.get("unit"), "frac": d.get("frac"), "traffic": traffic, "kernel": dom,
                "avg_ms": d["avg_ms"], "work_per_launch": d.get("work_per_launch")}

    cpu = None
    check = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(case, args.cpu_seconds)
        log(f"[bench] oracle {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")
        # the same sample checks the GPU output of the last timed step
        import numpy as np
        rows, yr, den = cpu.pop("_rows"), cpu.pop("_y"), cpu.pop("_den")
        idx = torch.as_tensor(rows, device=dev, dtype=torch.long)
        yg = out.reshape(-1, case.o).index_select(0, idx).double().cpu().numpy()
        rel = np.abs(yg - yr) / np.where(den > 0, den, 1.0)
        check = {"outputs": int(rel.size), "max_err_over_sum_abs": float(rel.max()),
                 "mean_err_over_sum_abs": float(rel.mean()), "tol": 2e-5, "within_tol": bool(rel.max() <= 2e-5)}
        log(f"[bench] oracle check: max |y - y_ref| / sum|x||w| = {check['max_err_over_sum_abs']:.3g}")

    configs = None
    if not args.no_configs:
        log("[bench] timing the other workloads")
        configs = run_configs(dev, (case, x, w, out))

    line = {
        "metric": "conv fwd TFLOP/s (2*N*OH*OW*O*C*KH*KW/s) and % of roofline",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        # GPU span of each timed step (first kernel to the end of the last), from the library's events
        "ms_per_step_median": spans[len(spans) // 2],
        "ms_per_step_min": spans[0],
        "higher_is_better": True,
        "scaling": "weak",
        # against the reported baseline: the fp64 oracle timed on this host's cores in the same run
        "vs_baseline": value / cpu["value"] if cpu else None,
        "vs_baseline_basis": "cpu_baseline (the fp64 oracle on this host, same run)",
        # the tiling page's ~310 ms Winograd time for this conv on an M2 Max: another machine's, context only
        "context": {"page_m2_max_tflops": PAGE_BASELINE_TFLOPS, "ratio": value / PAGE_BASELINE_TFLOPS},
        "dtype": "f32",
        "data": "synthetic (seeded numpy PCG64: x ~ U[-1,1], w ~ N(0, 1/(9C)))",
        "config": {"workload": f"conv2d fp32 NHWC N={case.n}, 512x512, C=192 -> O=96, 3x3, stride 1, pad 1",
                   "algo": plan.algo_name, "tile_batch": plan.tile_batch, "n_tiles": plan.n_tiles,
                   "ws_limit_bytes": int(ws_limit), "workspace_bytes": int(plan.workspace_bytes),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "stages": stages,
        "cpu_baseline": cpu,
        "oracle_check": check,
        "configs": configs,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
