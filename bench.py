#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the whole hot path (one fused forward kernel) over the
workload's seeded synthetic inputs, already resident in HBM.  Before the W
warmup and K timed steps, an untimed clock-settle phase of fixed length
(--settle-ms, default 250 ms of back-to-back steps) brings the chip to the
clock it holds under this load; the line reports it.  Prints ONE JSON
line: throughput in TFLOP/s (FLOPs = 2*B*Hq*Lq*Lk*(d_qk+d_v), halved when
causal), the roofline object of the kernel (per-launch duration from HIP
events on the launch stream), and the CPU oracle timed on a bounded sample of
the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (bf16, 1 GPU) and % of MI355X dense bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0      # MI355X published HBM3E bandwidth
CSRC = os.path.join(ROOT, "exact_attention_forward_02_amd", "csrc")
KERNEL_SOURCE = os.path.join(CSRC, "attn_fwd_kernel.hip")
DECODE_SOURCE = os.path.join(CSRC, "attn_decode_kernel.hip")
BWD_SOURCE = os.path.join(CSRC, "attn_bwd_kernel.hip")


def kernel_source_digest(path: str = KERNEL_SOURCE) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str, kernel: str = "attn_fwd", source: str = KERNEL_SOURCE):
    """HBM bytes per launch from committed rocprofv3 counter runs
    (profiles/traffic_<kernel>_<workload>.json), if they were taken on the
    current kernel source; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path, encoding="utf-8") as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256") != kernel_source_digest(source):
        return None
    return rec.get("hbm_bytes_per_launch")


def host_threads() -> int:
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


SETTLE_MS = 250.0  # default length of the untimed clock-settle phase


def settle(launch, settle_ms: float) -> dict:
    """Untimed clock-settle phase before the warmup: the step's launches run back
    to back, in batches of 8 with a synchronisation after each, until
    `settle_ms` of wall time have passed.  The MI355X raises its clock over the
    first tens of milliseconds of load; this makes the timed steps, whatever
    their number, run at the clock the chip holds under this load.  Its length
    is fixed in time (the launch count it took is reported)."""
    import torch

    n = 0
    t0 = time.perf_counter()
    if settle_ms > 0:
        while (time.perf_counter() - t0) * 1e3 < settle_ms:
            for _ in range(8):
                launch()
            n += 8
            torch.cuda.synchronize()
    return {"ms": settle_ms, "launches": n,
            "seconds": round(time.perf_counter() - t0, 4)}


def cpu_baseline(w, q, k, v, target_s: float = 12.0):
    """Oracle (fp64, as it stands) on a bounded random sample of query rows."""
    import oracle
    from exact_attention_forward_02_amd.inputs import sample_rows

    orc = oracle.load()
    threads = host_threads()
    per_row_flops = 2.0 * w.Lk * (w.dqk + w.dv)  # non-causal rows see every key
    if w.causal:
        per_row_flops /= 2.0  # average visible keys under the causal mask
    total_rows = w.B * w.Hq * w.Lq
    probe = sample_rows(w.B, w.Hq, w.Lq, 8 * threads, seed=12345).numpy()
    t0 = time.perf_counter()
    orc.attn_rows(q, k, v, causal=w.causal, rows=probe, threads=threads)
    t_probe = time.perf_counter() - t0
    n = int(min(total_rows, max(len(probe), len(probe) * target_s / max(t_probe, 1e-6))))
    rows = sample_rows(w.B, w.Hq, w.Lq, n, seed=54321).numpy()
    t0 = time.perf_counter()
    o_ref, l_ref = orc.attn_rows(q, k, v, causal=w.causal, rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    if dt < 0.5 * target_s and n < total_rows:
        # the small probe overstates the per-row cost (thread start-up): size
        # the sample once more from this measured one
        n = int(min(total_rows, n * target_s / max(dt, 1e-6)))
        rows = sample_rows(w.B, w.Hq, w.Lq, n, seed=54321).numpy()
        t0 = time.perf_counter()
        o_ref, l_ref = orc.attn_rows(q, k, v, causal=w.causal, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
    # exact FLOPs of the sampled rows
    if w.causal:
        off = w.Lk - w.Lq
        i = rows % w.Lq
        keys = (i + off + 1).clip(0, w.Lk)
        flops = float((2.0 * keys * (w.dqk + w.dv)).sum())
    else:
        flops = per_row_flops * len(rows)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{len(rows)} of {total_rows} query rows of {w.name} drawn at random "
                  f"(seeded), fp64 materialised softmax, {dt:.1f} s",
        "seconds": dt,
        # the oracle's rows, for the parity summary of the timed output
        "_rows": rows, "_o": o_ref, "_lse": l_ref,
    }


def parity_summary(o_gpu, lse_gpu, o_ref, lse_ref) -> dict:
    """max / mean |dO| and max |dlse| of GPU rows against the oracle's (rows
    without a visible key must be O = 0, lse = -inf)."""
    import numpy as np

    empty = np.isneginf(lse_ref)
    full = ~empty
    err = np.abs(o_gpu[full] - o_ref[full])
    return {
        "rows": int(len(lse_ref)),
        "o_max": float(err.max()) if err.size else 0.0,
        "o_mean": float(err.mean()) if err.size else 0.0,
        "lse_max": float(np.abs(lse_gpu[full] - lse_ref[full]).max()) if full.any() else 0.0,
        "empty_rows_exact": bool(np.all(o_gpu[empty] == 0.0) and np.all(np.isneginf(lse_gpu[empty]))),
    }


HIP_ATTR_CLOCK_RATE = 5  # hipDeviceAttributeClockRate: peak clock in kHz


def peak_clock_khz(index: int):
    """The device's peak clock from the HIP runtime already loaded in this
    process (hipDeviceGetAttribute), or None.  Only a runtime that is already
    mapped is used, so no second copy of it is ever loaded."""
    import ctypes

    path = None
    try:
        with open("/proc/self/maps", encoding="utf-8") as f:
            for line in f:
                if "libamdhip64" in line and "/" in line:
                    path = line[line.index("/"):].strip()
                    break
    except OSError:
        return None
    if path is None:
        return None
    try:
        hip = ctypes.CDLL(path, mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
    except OSError:
        return None
    value = ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(value), HIP_ATTR_CLOCK_RATE, int(index)) != 0:
        return None
    return value.value


def environment(dev) -> dict:
    import torch

    prop = torch.cuda.get_device_properties(dev)
    khz = peak_clock_khz(dev.index or 0)
    cus = prop.multi_processor_count
    env = {"device": prop.name, "arch": prop.gcnArchName, "compute_units": cus,
           "peak_clock_mhz": khz / 1000.0 if khz else None,
           "torch": torch.__version__, "hip": getattr(torch.version, "hip", None)}
    if khz:
        # dense bf16 MFMA: 4 SIMDs per CU, 1024 flop per SIMD per clock
        # (v_mfma_f32_32x32x16_bf16: 32768 flop in 32 cycles)
        env["bf16_peak_formula"] = (f"{cus} CU x 4 SIMD x 1024 flop/clk x {khz / 1e6:.2f} GHz = "
                                    f"{cus * 4 * 1024 * khz * 1e3 / 1e15:.3f} PFLOP/s "
                                    f"(published {PEAK_BF16_TFLOPS / 1000:.1f})")
    return env


COPY_BYTES = 1 << 30  # bytes read (and written) per calibration launch


def copy_calibration() -> int:
    """torch.neg over 1 GiB of bf16: one elementwise kernel reading COPY_BYTES
    and writing COPY_BYTES, launched three times."""
    import torch

    dev = torch.device("cuda:0")
    x = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": COPY_BYTES,
                                           "bytes_written": COPY_BYTES, "launches": 3}}))
    return 0


def bench_split(args, w, qd, kd, vd) -> int:
    """The split-key path: per step one attn_fwd_split launch (the dominant
    kernel, timed alone with HIP events on its stream) and one attn_merge.
    Few query rows make it bound by reading K and V: its roofline is HBM."""
    import torch

    from exact_attention_forward_02_amd import attn_fwd_split, attn_merge, library

    n = args.splits
    dev = qd.device
    stream = torch.cuda.current_stream(dev)
    o_part = torch.empty((n, w.B, w.Hq, w.Lq, w.dv), dtype=torch.float32, device=dev)
    lse_part = torch.empty((n, w.B, w.Hq, w.Lq), dtype=torch.float32, device=dev)
    o = torch.empty((w.B, w.Hq, w.Lq, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device=dev)

    # one checked call through the binding, then the same C-ABI entry points
    # called directly with the prepared arguments, so that the host enqueues
    # faster than these short kernels run and no host time falls between a
    # launch and its events
    attn_fwd_split(qd, kd, vd, n, causal=w.causal, o_part=o_part, lse_part=lse_part,
                   stream=stream)
    attn_merge(o_part, lse_part, out=o, lse=lse, stream=stream)
    lib = library()
    scale = 1.0 / math.sqrt(w.dqk)
    a_split = (qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_part.data_ptr(), lse_part.data_ptr(),
               w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.dqk, w.dv, int(w.causal), scale, n,
               stream.cuda_stream)
    a_merge = (o_part.data_ptr(), lse_part.data_ptr(), o.data_ptr(), lse.data_ptr(), n,
               w.B * w.Hq * w.Lq, w.dv, stream.cuda_stream)
    codes = []

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        codes.append(lib.attn_fwd_split(*a_split))
        if ev is not None:
            ev[1].record(stream)
        codes.append(lib.attn_merge(*a_merge))
        if ev is not None:
            ev[2].record(stream)

    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if any(c != 0 for c in codes):
        raise RuntimeError(f"split path returned status {sorted(set(codes))}")
    split_ms = [e[0].elapsed_time(e[1]) for e in evs]
    merge_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_split = sum(split_ms) / len(split_ms)
    ms_merge = sum(merge_ms) / len(merge_ms)
    flops = w.flops()
    # algorithmic bytes of the split kernel: Q, K, V read once, every split's
    # fp32 state written once
    rows = w.B * w.Hq * w.Lq
    split_bytes = (2 * (w.B * w.Hq * w.Lq * w.dqk + w.B * w.Hkv * w.Lk * (w.dqk + w.dv))
                   + n * rows * (4 * w.dv + 4))
    merge_bytes = n * rows * (4 * w.dv + 4) + rows * (2 * w.dv + 4)
    gbs = split_bytes / (ms_split * 1e-3) / 1e9
    decode = w.Lq * (w.Hq // w.Hkv) <= 16
    result = {
        "metric": METRIC,
        "value": round(flops * args.steps / wall / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settled,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq,
                   "Lk": w.Lk, "d_qk": w.dqk, "d_v": w.dv, "causal": w.causal,
                   "splits": n, "flops_per_step": flops},
        "roofline": {
            "bound": "hbm",
            "achieved": round(gbs, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": (measured_traffic(w.name, "attn_decode", DECODE_SOURCE) if decode
                        else None),
            "kernel": "attn_decode_kernel" if decode else "attn_fwd_kernel (split)",
            "bytes_per_launch": split_bytes,
            "ms_per_launch": round(ms_split, 4),
            "ms_per_launch_min": round(min(split_ms), 4),
            "ms_per_launch_max": round(max(split_ms), 4),
            "merge_ms_per_launch": round(ms_merge, 4),
            "merge_gbs": round(merge_bytes / (ms_merge * 1e-3) / 1e9, 1),
        },
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_backward(args, w, qd, kd, vd) -> int:
    """The backward pass: per step one attn_bwd call (D, then dK/dV, then dQ;
    with d_qk = 192, dV and dK in two passes) on the forward's o and lse.  Its
    algorithmic work is the five products of the backward (S recomputed, dP,
    dV, dK, dQ): 2 * pairs * (3 d_qk + 2 d_v) FLOPs, 2.5 times the forward's
    when d_qk = d_v."""
    import torch

    from exact_attention_forward_02_amd import attn_bwd, attn_fwd

    dev = qd.device
    stream = torch.cuda.current_stream(dev)
    g = torch.Generator().manual_seed(w.seed + 1)
    dout = torch.randn((w.B, w.Hq, w.Lq, w.dv), generator=g).to(torch.bfloat16).to(dev)
    o, lse = attn_fwd(qd, kd, vd, causal=w.causal, stream=stream)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    delta = torch.empty_like(lse)

    def step():
        attn_bwd(qd, kd, vd, o, lse, dout, causal=w.causal, dq=dq, dk=dk, dv=dv, delta=delta,
                 stream=stream)

    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_launch = sum(launch_ms) / len(launch_ms)
    # the five products: S and dK, dQ over d_qk, dP and dV over d_v (2.5 times the
    # forward's FLOPs when d_qk = d_v)
    flops = w.flops() * (3 * w.dqk + 2 * w.dv) / (w.dqk + w.dv)
    value = flops * args.steps / wall / 1e12
    achieved = flops / (ms_launch * 1e-3) / 1e12
    result = {
        "metric": "attention bwd TFLOP/s (bf16, 1 GPU) and % of MI355X dense bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settled,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq,
                   "Lk": w.Lk, "d_qk": w.dqk, "d_v": w.dv, "causal": w.causal,
                   "pass": "backward", "flops_per_step": flops},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(w.name, "attn_bwd", BWD_SOURCE),
            "kernel": "attn_bwd (D, dK/dV and dQ kernels)",
            "ms_per_launch": round(ms_launch, 4),
            "ms_per_launch_min": round(min(launch_ms), 4),
            "ms_per_launch_max": round(max(launch_ms), 4),
        },
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_varlen(args, w) -> int:
    """A packed variable-length batch: the host planner runs once per batch
    (its time is reported as plan_ms, outside the steps), then each step is one
    attn_fwd_varlen launch on the uploaded plan."""
    import numpy as np
    import torch

    import oracle
    from exact_attention_forward_02_amd import attn_fwd_varlen, varlen_plan
    from exact_attention_forward_02_amd.inputs import varlen_workload_qkv

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v, cu_q, cu_k = varlen_workload_qkv(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    t0 = time.perf_counter()
    plan_host = varlen_plan(cu_q, cu_k, w.Hq, w.Hkv, w.causal)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plan = torch.from_numpy(plan_host).to(dev)
    T = q.shape[0]
    o = torch.empty((T, w.Hq, w.dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.Hq, T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        attn_fwd_varlen(qd, kd, vd, cu_q, cu_k, causal=w.causal, plan=plan, out=o, lse=lse,
                        stream=stream)

    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_launch = sum(launch_ms) / len(launch_ms)
    flops = w.flops()
    value = flops * args.steps / wall / 1e12
    achieved = flops / (ms_launch * 1e-3) / 1e12
    lens = w.lengths()
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settled,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "total_tokens": w.total, "n_seq": len(lens),
                   "seq_lens": lens, "Hq": w.Hq, "Hkv": w.Hkv, "d_qk": w.dqk, "d_v": w.dv,
                   "causal": w.causal, "layout": "thd", "flops_per_step": flops,
                   "tile_records": int(plan_host.shape[0]), "plan_ms": round(plan_ms, 3)},
        "env": environment(dev),
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(w.name),
            "kernel": "attn_fwd_kernel (varlen)",
            "ms_per_launch": round(ms_launch, 4),
            "ms_per_launch_median": round(sorted(launch_ms)[len(launch_ms) // 2], 4),
            "ms_per_launch_min": round(min(launch_ms), 4),
            "ms_per_launch_max": round(max(launch_ms), 4),
        },
    }
    if not args.no_cpu_baseline:
        orc = oracle.load()
        threads = host_threads()
        g = torch.Generator().manual_seed(54321)
        n_rows = min(w.Hq * T, 10000 * threads)  # about 10 s of fp64 work
        rows = torch.randperm(w.Hq * T, generator=g)[:n_rows].numpy()
        t0 = time.perf_counter()
        o_ref, l_ref = orc.attn_varlen(q, k, v, cu_q, cu_k, causal=w.causal, rows=rows,
                                       threads=threads)
        dt = time.perf_counter() - t0
        # exact FLOPs of the sampled rows: each sees its visible keys
        cq = np.asarray(cu_q)
        tok = rows % T
        seq = np.searchsorted(cq, tok, side="right") - 1
        L = (cq[seq + 1] - cq[seq])
        i = tok - cq[seq]
        keys = (i + 1) if w.causal else L
        rflops = float((2.0 * keys * (w.dqk + w.dv)).sum())
        result["cpu_baseline"] = {
            "value": float(f"{rflops / dt / 1e12:.4g}"), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{len(rows)} of {w.Hq * T} query rows of {w.name} drawn at random "
                      f"(seeded), fp64 materialised softmax, {dt:.1f} s"}
        ridx = torch.from_numpy(rows).to(dev)
        og = o.permute(1, 0, 2).reshape(-1, w.dv).index_select(0, ridx)
        lg = lse.reshape(-1).index_select(0, ridx)
        result["parity"] = parity_summary(og.double().cpu().numpy(), lg.double().cpu().numpy(),
                                          o_ref, l_ref)
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="length of the untimed clock-settle phase before the warmup, in ms "
                         "of back-to-back steps (0: none)")
    ap.add_argument("--workload", default="mha_l2k")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain copy kernel of known size (3 launches) to "
                         "calibrate the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--dtype", choices=("bf16", "fp16"), default="bf16",
                    help="element type of q, k, v and o (fp16 runs through attn_fwd_ex)")
    ap.add_argument("--layout", choices=("bhsd", "bshd"), default="bhsd",
                    help="storage of q, k, v and o: [B, H, L, d] or [B, S, H, d] (the "
                         "latter runs through attn_fwd_ex with strides)")
    ap.add_argument("--splits", type=int, default=0,  # decode_l32k is timed with 4
                    help="time the split-key path instead (attn_fwd_split with this many "
                         "key splits, then attn_merge); reported against the HBM roofline")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (attn_bwd on the forward's o and lse) "
                         "instead of the forward")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this kernel runs on a single MI355X and "
              "the multi-GPU path is not built; run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    from exact_attention_forward_02_amd import attn_fwd, attn_fwd_ex
    from exact_attention_forward_02_amd.inputs import WORKLOADS, workload_qkv

    if args.copy_calibration:
        return copy_calibration()
    from exact_attention_forward_02_amd.inputs import VARLEN_WORKLOADS

    if args.workload in VARLEN_WORKLOADS:
        return bench_varlen(args, VARLEN_WORKLOADS[args.workload])
    if args.workload not in WORKLOADS:
        print(f"unknown workload {args.workload}; choose from "
              f"{sorted(WORKLOADS) + sorted(VARLEN_WORKLOADS)}",
              file=sys.stderr)
        return 2
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q, k, v = workload_qkv(w)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    if args.splits > 0:
        return bench_split(args, w, qd, kd, vd)
    if args.backward:
        return bench_backward(args, w, qd, kd, vd)
    variant = args.dtype != "bf16" or args.layout != "bhsd"
    if variant:
        # the same draws, carried in the requested type and storage
        et = torch.float16 if args.dtype == "fp16" else torch.bfloat16
        q, k, v = (t.float().to(et) for t in (q, k, v))
        qd, kd, vd = (t.to(dev) for t in (q, k, v))
        if args.layout == "bshd":
            qd, kd, vd = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (qd, kd, vd))
            o = torch.empty((w.B, w.Lq, w.Hq, w.dv), dtype=et, device=dev).transpose(1, 2)
        else:
            o = torch.empty((w.B, w.Hq, w.Lq, w.dv), dtype=et, device=dev)
        fwd = attn_fwd_ex
    else:
        o = torch.empty((w.B, w.Hq, w.Lq, w.dv), dtype=torch.bfloat16, device=dev)
        fwd = attn_fwd
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        fwd(qd, kd, vd, causal=w.causal, out=o, lse=lse, stream=stream)

    settled = settle(step, args.settle_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_launch = sum(launch_ms) / len(launch_ms)
    ms_step = wall * 1e3 / args.steps
    import statistics

    flops = w.flops()
    value = flops * args.steps / wall / 1e12
    achieved = flops / (ms_launch * 1e-3) / 1e12
    # the stored counter record covers the default bf16 [B, H, L, d] run
    traffic = None if variant else measured_traffic(w.name)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settled,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq,
                   "Lk": w.Lk, "d_qk": w.dqk, "d_v": w.dv, "causal": w.causal,
                   "layout": args.layout, "flops_per_step": flops,
                   # the same count over the exact visible (query, key) pairs: under
                   # the causal mask it exceeds the halved convention by about 1/L
                   "flops_exact_pairs": 2.0 * w.B * w.Hq * w.valid_pairs() * (w.dqk + w.dv)},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": "attn_fwd_kernel",
            "ms_per_launch": round(ms_launch, 4),
            "ms_per_launch_median": round(statistics.median(launch_ms), 4),
            "ms_per_launch_min": round(min(launch_ms), 4),
            "ms_per_launch_max": round(max(launch_ms), 4),
        },
        "env": environment(dev),
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(w, q, k, v)
        cb.pop("seconds", None)
        cb["value"] = float(f"{cb['value']:.4g}")
        rows = torch.as_tensor(cb.pop("_rows"), dtype=torch.int64)
        o_ref, l_ref = cb.pop("_o"), cb.pop("_lse")
        og = o.contiguous().reshape(-1, w.dv).index_select(0, rows.to(dev))
        lg = lse.reshape(-1).index_select(0, rows.to(dev))
        result["cpu_baseline"] = cb
        # the timed launches' output on the oracle's rows (no assertion here:
        # the tests hold the bar)
        result["parity"] = parity_summary(og.double().cpu().numpy(), lg.double().cpu().numpy(),
                                          o_ref, l_ref)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
