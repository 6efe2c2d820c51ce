#!/usr/bin/env python3
"""Benchmark of the producer-fused NVFP4 activation quantizer on one MI355X.

One step = one pass of the fused RMSNorm + adaLN -> NVFP4 producer over the whole
63,240 x 7168 bf16 activation of an H3 block (34x60 latent tokens x 31 frames, 56 heads x
128), inputs resident in HBM, outputs: packed E2M1 codes + swizzled E4M3 scales.

Prints ONE JSON line:
  value      whole-job HBM throughput, algorithmic bytes / time per step (GB/s)
  roofline   the kernel's algorithmic GB/s (per-launch HIP events) against 8 TB/s peak,
             plus measured HBM traffic per launch from the committed rocprofv3 counter
             summary when it was taken on the current kernel sources (else null)
  stream_ceiling_GBps  a bench-side kernel (libnvfp4act_selftest.so) that moves the same
             bytes as a bf16 NVFP4 producer (2 B read, 0.5625 B written per element) with no
             arithmetic: what the memory system delivers for this mix
  cpu_baseline  the CPU oracle timed over the whole workload on every CPU this process may
             use, and on one thread
When one set of inputs and outputs is smaller than 512 MB (so that it could stay in the
256 MB Infinity Cache between steps) the steps rotate over enough copies to exceed it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused RMSNorm+adaLN→NVFP4 HBM GB/s & % of peak at 63,240×7168 bf16"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, vendor figure


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="rms_adaln_63240x7168")
    p.add_argument("--dynamic", action="store_true",
                   help="time the per-call (dynamic) amax form: amax pass + quantize pass")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0, help="rows of the oracle sample (0: all rows)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also time a device-to-device copy of the input (the HBM counter calibration)")
    return p.parse_args()


def cpu_share():
    """(CPUs this process may run on, CPUs its cgroup quota allows or None)."""
    avail = len(os.sched_getaffinity(0))
    quota = None
    try:
        q, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = max(1, int(int(q) // int(period)))
    except (OSError, ValueError):
        pass
    return avail, quota


def stream_ceiling(torch, wl, stream):
    """GB/s of the bench-side stream kernel over this workload's [m, k] shape, or None when
    the workload is not a single bf16 input of k <= 8192 columns quantized to NVFP4."""
    import ctypes
    if wl.kind not in ("rms_adaln", "quantize") or wl.k > 8192 or wl.k % 512:
        return None
    lib = ctypes.CDLL(os.path.join(ROOT, "nvfp4_activation_quantization_amd", "libnvfp4act_selftest.so"))
    fn, cols = lib.nvfp4act_selftest_stream, wl.k
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    fn.restype = ctypes.c_int
    x = torch.empty((wl.m, cols), dtype=torch.int16, device="cuda:0")
    x.fill_(0x3F80)
    codes = torch.empty((wl.m, wl.k // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty(((wl.m + 127) // 128 * 128, wl.k // 16), dtype=torch.uint8, device="cuda:0")

    def run():
        rc = fn(x.data_ptr(), wl.m, wl.k, codes.data_ptr(), scales.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("bench-side stream kernel returned %d" % rc)

    for _ in range(20):
        run()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for s, e in ev:
        s.record(stream)
        run()
        e.record(stream)
    torch.cuda.synchronize()
    ms = sum(s.elapsed_time(e) for s, e in ev) / len(ev)
    nbytes = wl.m * cols * 2 + wl.m * wl.k // 2 + (wl.m + 127) // 128 * 128 * (wl.k // 16)
    return nbytes / (ms * 1e-3) / 1e9


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "nvfp4_activation_quantization_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(csrc, "*"))):
        h.update(os.path.basename(path).encode())
        h.update(open(path, "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from profiles/traffic_<workload>.txt, if it was measured on
    the current kernel sources (its source_sha256 line), else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % workload)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return int(float(kv["fetch_bytes_per_launch"])) + int(float(kv["write_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def make_inputs(wl, torch, amax):
    import numpy as np
    dev = "cuda:0"

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    if wl.kind == "rms_adaln":
        x = up(wl.x())
        args = dict(x=x, weight=up(wl.weight()), table=up(wl.table()),
                    frame_idx=torch.from_numpy(wl.frame_idx()).to(dev))
    elif wl.kind == "residual_rms":
        def f32(a):
            return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)
        args = dict(x=f32(wl.h()), o=up(wl.o()), bias=up(wl.bias()), scale=f32(wl.residual_scale()),
                    gamma=f32(wl.gamma()))
    elif wl.kind == "rms_silu":
        args = dict(x=up(wl.x()), gamma=up(wl.weight()))
    elif wl.kind == "ln_fp8":
        sc, sh = wl.modulation()
        args = dict(x=up(wl.x()), scale=torch.from_numpy(sc).to(dev), shift=torch.from_numpy(sh).to(dev))
    elif wl.kind == "residual_adaln":
        args = dict(x=torch.from_numpy(wl.h()).to(dev), o=up(wl.o()), bias=up(wl.bias()), gate=up(wl.gate_table()),
                    weight=up(wl.weight()), table=up(wl.table()), frame_idx=torch.from_numpy(wl.frame_idx()).to(dev))
    else:
        args = dict(x=up(wl.x()))
        if wl.kind == "swiglu" and wl.bias_std > 0:
            args["bias"] = up(wl.bias())
    return args


def make_step(wl, a, nq, workloads, inp, amax, amax_dev, stream):
    """The step function of one input/output set: one launch of the workload's entry point."""
    import torch
    if wl.kind == "rms_silu":
        codes = torch.empty((wl.m, wl.k // 2), dtype=torch.uint8, device="cuda:0")
        scales = torch.empty((wl.m, wl.k // 16), dtype=torch.uint8, device="cuda:0")
    elif wl.kind == "ln_fp8":
        codes, scales = torch.empty((wl.m, wl.k), dtype=torch.uint8, device="cuda:0"), None
    else:
        codes, scales = nq.new_quantized(wl.m, wl.k, "cuda:0")

    if wl.kind == "ln_fp8":
        act_scale = workloads.fp8_act_scale(wl.name)
        if a.dynamic:
            def step():
                nq.ln_adaln_fp8_dynamic(inp["x"], inp["scale"], inp["shift"], wl.eps, act_scale_out=amax_dev,
                                        codes=codes, stream=stream)
        else:
            def step():
                nq.ln_adaln_fp8(inp["x"], inp["scale"], inp["shift"], wl.eps, act_scale, codes=codes, stream=stream)
    elif wl.kind == "rms_silu":
        if a.dynamic:
            def step():
                nq.rms_silu_nvfp4_dynamic(inp["x"], inp["gamma"], wl.eps, amax_out=amax_dev, codes=codes,
                                          scales=scales, stream=stream)
        else:
            def step():
                nq.rms_silu_nvfp4(inp["x"], inp["gamma"], wl.eps, amax, codes=codes, scales=scales, stream=stream)
        nq.init()
    elif wl.kind == "residual_adaln":
        # the stream is updated in place every step (the same work each time)
        residual = (inp["o"], inp["bias"], inp["gate"])
        fold_args = (inp["x"], inp["weight"], inp["table"], inp["frame_idx"], wl.eps)
        if a.dynamic:
            def step():
                nq.residual_rms_adaln_nvfp4_dynamic(*fold_args, residual=residual, amax_out=amax_dev, codes=codes,
                                                    scales=scales, stream=stream)
        else:
            def step():
                nq.residual_rms_adaln_nvfp4(*fold_args, amax, residual=residual, codes=codes, scales=scales,
                                            stream=stream)
    elif wl.kind == "residual_rms":
        # the stream is updated in place every step (the same work each time)
        residual = (inp["o"], inp["bias"], inp["scale"])
        if a.dynamic:
            def step():
                nq.residual_rms_nvfp4_dynamic(inp["x"], inp["gamma"], wl.eps, residual=residual, amax_out=amax_dev,
                                              codes=codes, scales=scales, stream=stream)
        else:
            def step():
                nq.residual_rms_nvfp4(inp["x"], inp["gamma"], wl.eps, amax, residual=residual, codes=codes,
                                      scales=scales, stream=stream)
    elif wl.kind == "rms_adaln" and a.dynamic:
        def step():
            nq.rms_adaln_nvfp4_dynamic(inp["x"], inp["weight"], inp["table"], inp["frame_idx"], wl.eps,
                                       amax_out=amax_dev, codes=codes, scales=scales, stream=stream)
    elif wl.kind == "rms_adaln":
        def step():
            nq.rms_adaln_nvfp4(inp["x"], inp["weight"], inp["table"], inp["frame_idx"], wl.eps, amax,
                               codes=codes, scales=scales, stream=stream)
    elif wl.kind == "quantize" and a.dynamic:
        def step():
            nq.nvfp4_quantize_dynamic(inp["x"], amax_out=amax_dev, codes=codes, scales=scales, stream=stream)
    elif wl.kind == "quantize":
        def step():
            nq.nvfp4_quantize(inp["x"], amax, codes=codes, scales=scales, stream=stream)
    elif (wl.bias_std > 0 or wl.interleaved) and a.dynamic:
        def step():
            nq.swiglu_packed_nvfp4_dynamic(inp["x"], bias=inp.get("bias"), interleaved=wl.interleaved,
                                           amax_out=amax_dev, codes=codes, scales=scales, stream=stream)
        nq.init()
    elif wl.bias_std > 0 or wl.interleaved:
        def step():
            nq.swiglu_packed_nvfp4(inp["x"], amax, bias=inp.get("bias"), interleaved=wl.interleaved, codes=codes,
                                   scales=scales, stream=stream)
        nq.init()
    elif a.dynamic:
        def step():
            nq.swiglu_nvfp4_dynamic(inp["x"], amax_out=amax_dev, codes=codes, scales=scales, stream=stream)
        nq.init()
    else:
        def step():
            nq.swiglu_nvfp4(inp["x"], amax, codes=codes, scales=scales, stream=stream)
        nq.init()
    return step


def main():
    a = parse()
    if a.gpus != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (rows are "
              "independent, so each GPU would quantize its own range of rows).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nvfp4_activation_quantization_amd as nq
    import workloads

    wl = workloads.get(a.workload)
    amax = workloads.calibration_amax(wl.name)
    torch.cuda.set_device(0)
    inp = make_inputs(wl, torch, amax)
    amax_dev = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()

    # input/output sets: enough that one step's working set does not stay in the 256 MB
    # Infinity Cache from one step to the next
    working_set = wl.algorithmic_bytes()
    n_sets = 1 if working_set >= (512 << 20) else min(8, -(-(512 << 20) // working_set))
    steps_fns = []
    for set_i in range(n_sets):
        inp_i = inp if set_i == 0 else {key: v.clone() for key, v in inp.items()}
        steps_fns.append(make_step(wl, a, nq, workloads, inp_i, amax, amax_dev, stream))
    torch.cuda.synchronize()
    step_count = [0]

    def step():
        steps_fns[step_count[0] % n_sets]()
        step_count[0] += 1

    # GPU clock warm-up (untimed): a fresh process runs the first tens of milliseconds
    # of work at a lower clock, so run the step for ~0.3 s before the W warmup steps.
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.3:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, per-launch events on the launch stream
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region0.record(stream)
    for i in range(a.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    region1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = region0.elapsed_time(region1)
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kernel_ms = float(np.mean(per_launch_ms))
    ms_per_step = region_ms / a.steps

    # the per-call form reads the input twice (the amax pass, then the quantize pass)
    reread = (4 + 2) * wl.m * wl.k if wl.kind.startswith("residual") else 2 * wl.m * wl.in_cols
    alg_bytes = wl.algorithmic_bytes() + (reread if a.dynamic else 0)
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9

    # practical ceiling for context: the same bytes moved with no arithmetic
    ceiling = stream_ceiling(torch, wl, stream)
    copy_gbps = None
    if a.copy_calibration:
        # a device-to-device copy of the input: the kernel the HBM counters are scaled by
        x = inp["x"]
        dst = torch.empty_like(x)
        for _ in range(3):
            dst.copy_(x)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        for _ in range(10):
            dst.copy_(x)
        c1.record(stream)
        torch.cuda.synchronize()
        copy_gbps = 2 * x.numel() * x.element_size() / (c0.elapsed_time(c1) / 10 * 1e-3) / 1e9
        del dst

    traffic = None if a.dynamic else measured_traffic(wl.name)

    out = {
        "metric": (METRIC if wl.name == "rms_adaln_63240x7168" and not a.dynamic
                   else "NVFP4 producer HBM GB/s (%s%s)" % (wl.name, ", per-call amax" if a.dynamic else "")),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "rows": wl.m, "hidden": wl.k,
                   "frames": wl.frames if wl.frames else None,
                   "algorithmic_bytes_per_step": alg_bytes,
                   "working_set_bytes": working_set, "rotated_sets": n_sets,
                   ("act_scale" if wl.kind == "ln_fp8" else "global_amax"):
                       "per-call (device amax pass)" if a.dynamic
                       else (workloads.fp8_act_scale(wl.name) if wl.kind == "ln_fp8" else amax)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic},
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBPS, 2),
        "rows_per_s": round(wl.m / (ms_per_step * 1e-3), 1),
        "kernel_us": round(kernel_ms * 1e3, 2),
        "kernel_us_median": round(float(np.median(per_launch_ms)) * 1e3, 2),
        "kernel_us_min": round(float(np.min(per_launch_ms)) * 1e3, 2),
        "stream_ceiling_GBps": None if ceiling is None else round(ceiling, 1),
        "wall_s": round(wall, 3),
    }
    if ceiling is not None:
        out["roofline"]["frac_of_stream_ceiling"] = round(achieved / ceiling, 4)
    if copy_gbps is not None:
        out["copy_GBps"] = round(copy_gbps, 1)

    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, amax, a.cpu_rows or wl.m, np)
    print(json.dumps(out), flush=True)


def cpu_baseline(wl, amax, rows, np):
    """The CPU oracle (unchanged) on the first `rows` rows of the workload (all rows by
    default), split into contiguous row blocks over every CPU this process may use (rows are
    independent), then the same rows on one thread."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    avail, quota = cpu_share()
    threads = max(1, min(avail, quota) if quota else avail)
    rows = min(rows, wl.m)
    sel = np.arange(rows)
    x = wl.x_rows(sel) if not wl.kind.startswith("residual") else None
    if wl.kind == "ln_fp8":
        import workloads
        sc, sh = wl.modulation()
        act_scale = workloads.fp8_act_scale(wl.name)

        def part(se):
            s, e = se
            oracle.ln_adaln_fp8_rows(x[s:e], sc, sh, wl.eps, act_scale=act_scale, want_y=False)
    elif wl.kind == "rms_silu":
        gamma = wl.weight()
        oracle.silu_table_f16()

        def part(se):
            s, e = se
            oracle.rms_silu_rows(x[s:e], gamma, wl.eps, amax)
    elif wl.kind == "residual_adaln":
        x, o = wl.h_rows(sel), wl.o_rows(sel)
        fold = (wl.bias(), wl.gate_table(), wl.weight(), wl.table())
        idx = wl.frame_idx(sel)

        def part(se):
            s, e = se
            oracle.residual_rms_adaln_rows(x[s:e], o[s:e], *fold, idx[s:e], wl.eps, amax)
    elif wl.kind == "residual_rms":
        x, o = wl.h_rows(sel), wl.o_rows(sel)
        bias, scale, gamma = wl.bias(), wl.residual_scale(), wl.gamma()

        def part(se):
            s, e = se
            oracle.residual_rms_rows(x[s:e], o[s:e], bias, scale, gamma, wl.eps, amax)
    elif wl.kind == "rms_adaln":
        w, table, idx = wl.weight(), wl.table(), wl.frame_idx(sel)

        def part(se):
            s, e = se
            oracle.rms_adaln_rows(x[s:e], w, table, idx[s:e], wl.eps, amax)
    elif wl.kind == "quantize":
        def part(se):
            s, e = se
            oracle.quantize_rows(x[s:e], amax)
    elif wl.bias_std > 0 or wl.interleaved:
        oracle.silu_table()
        bias = wl.bias()

        def part(se):
            s, e = se
            oracle.swiglu_packed_rows(x[s:e], bias, wl.interleaved, amax)
    else:
        oracle.silu_table()

        def part(se):
            s, e = se
            oracle.swiglu_rows(x[s:e, :wl.k], x[s:e, wl.k:], amax)
    step = (rows + 4 * threads - 1) // (4 * threads)
    blocks = [(s, min(rows, s + step)) for s in range(0, rows, step)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(part, blocks))
    dt = time.perf_counter() - t0
    # the same rows on one thread
    t1 = time.perf_counter()
    part((0, rows))
    dt1 = time.perf_counter() - t1
    bytes_per_row = wl.algorithmic_bytes() / wl.m
    return {"value": round(rows * bytes_per_row / dt / 1e9, 4), "unit": "GB/s", "cores": threads,
            "threads": threads, "cores_available": avail, "cpu_quota": quota,
            "kind": "oracle", "rows_per_s": round(rows / dt, 1), "seconds": round(dt, 3),
            "single_thread_seconds": round(dt1, 3), "single_thread_rows_per_s": round(rows / dt1, 1),
            "single_thread_value": round(rows * bytes_per_row / dt1 / 1e9, 5), "cpu_model": cpu_model(),
            "sample": "%s %d rows of %s on %d threads (contiguous row blocks), then the same rows on one thread"
                      % ("all" if rows == wl.m else "first", rows, wl.name, threads)}


def cpu_model() -> str:
    """The host CPU: /proc/cpuinfo's model name with its family / model / stepping numbers
    (a virtual machine may shorten the name), and the socket / core counts lscpu reports."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = line.split(":", 1)
                fields.setdefault(k.strip(), v.strip())
    except OSError:
        pass
    desc = "%s (family %s, model %s, stepping %s)" % (fields.get("model name", "unknown"), fields.get("cpu family", "?"),
                                                    fields.get("model", "?"), fields.get("stepping", "?"))
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        info = dict(l.split(":", 1) for l in out.splitlines() if ":" in l)
        extra = [("Socket(s)", "sockets"), ("Core(s) per socket", "cores/socket"), ("Thread(s) per core", "threads/core"),
                 ("CPU(s)", "cpus")]
        desc += ", " + ", ".join("%s %s" % (name, info[key].strip()) for key, name in extra if key in info)
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    return desc


if __name__ == "__main__":
    main()
