#!/usr/bin/env python3
"""Benchmark: attention forward TFLOP/s on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]

One step is one fa_fwd call over the whole workload (every query row of every
head): the full hot path, one kernel launch.  Inputs are seeded synthetic
tensors already resident in HBM when the timed region starts.  W untimed steps,
then exactly K timed steps between two device synchronisations.

Before the W warm-up steps the kernel runs back to back for a fixed stretch
of wall time (``--precondition-seconds``, reported under ``preconditioning``):
the GPU raises its clock over the first tens of milliseconds of sustained
matrix work, and a handful of warm-up launches alone would time that ramp.

Printed: one JSON line (rank 0, the only rank).  ``value`` is 4*B*Hq*N^2*d
(halved when causal) per step over the timed wall time, in TFLOP/s.
``roofline`` prices the kernel's average launch duration, measured with HIP
events on the stream it runs on, against MI355X's dense bf16 MFMA peak; the
first and last five launch times show any drift within the timed steps.
``clock`` is the shader clock of one extra launch after the timed loop, read
from the kernel's own per-wave cycle and real-time counters.
``cpu_baseline`` times the fp64 oracle on a bounded, seeded sample of the same
workload's query rows on this host's cores and compares those rows with the
GPU output.
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


def metric_for(w) -> str:
    """The forward metric's name for this workload's dtype, sizes and mask; for the
    bench workload it is exactly the headline metric's."""
    mask = "causal" if w.causal else "non-causal"
    gqa = " GQA %d/%d" % (w.Hq, w.Hkv) if w.Hq != w.Hkv else ""
    return "attention fwd TFLOP/s (and %% of MFMA peak) at %s N=%d d=%d %s%s" % (w.dtype, w.N, w.d, mask, gqa)


# MI355X published dense peaks (no sparsity): 256 CUs at 2.4 GHz.
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3}
PEAK_HBM_GBPS = 8000.0

KERNEL_SOURCES = {
    "bf16": "flashattention_online_softmax_fwd_amd/csrc/fa_fwd_mfma16.hip",
    "f16": "flashattention_online_softmax_fwd_amd/csrc/fa_fwd_mfma16.hip",
    # the d = 128 forward of 16-bit inputs: 64 rows per wave, its key loop generated as assembly
    "w64": "flashattention_online_softmax_fwd_amd/csrc/fa_fwd_w64.hip",
    "f32": "flashattention_online_softmax_fwd_amd/csrc/fa_fwd_f32.hip",
    "merge": "flashattention_online_softmax_fwd_amd/csrc/fa_merge.hip",
    "softmax": "flashattention_online_softmax_fwd_amd/csrc/fa_softmax.hip",
    "bwd": "flashattention_online_softmax_fwd_amd/csrc/fa_bwd_mfma16.hip",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
SQ_FILE = os.path.join(ROOT, "profiles", "sq_counters.json")


def kernel_hash(source: str) -> str:
    """SHA-256 of the kernel's source file and the flags it is compiled with."""
    from flashattention_online_softmax_fwd_amd import build

    path = KERNEL_SOURCES[source]
    with open(os.path.join(ROOT, path), "rb") as f:
        data = f.read()
    if source == "w64":   # the generated key loop is part of the kernel
        with open(os.path.join(ROOT, os.path.dirname(path), "fa_fwd_kloop.inc"), "rb") as f:
            data += f.read()
    flags = " ".join(build.device_flags(os.path.basename(path))).encode()
    return hashlib.sha256(data + b"\0" + flags).hexdigest()


def forward_kernel(w, simds=1024):
    """(KERNEL_SOURCES key, kernel name) of the forward the library dispatches for ``w`` by
    default: fp32 has its own kernel; 16-bit inputs run the 64-rows-per-wave kernel when its
    waves cover every SIMD (``simds`` of the device), in 256-row workgroups (4 waves) when the
    grid holds at least 512 of them and in 128-row workgroups (2 waves) otherwise, and the
    32-rows-per-wave kernel (fwd16_kernel, 128-row workgroups) for fewer rows."""
    if w.dtype == "f32":
        return "f32", "fa::fwd_f32_kernel"
    units = w.B * w.Hq
    tname = "__bf16" if w.dtype == "bf16" else "_Float16"
    if units * ((w.N + 63) // 64) < simds:
        return w.dtype, "fa::fwd16_kernel<%s, %d, 128, 64, %s, false>" % (tname, w.d, "true" if w.causal else "false")
    nw = 4 if units * ((w.N + 255) // 256) >= 512 else 2
    return "w64", "fa::fwd_w64_kernel<%s, %s, %d, %d>" % (tname, "true" if w.causal else "false", nw, w.d)


def device_simds():
    import torch

    return 4 * torch.cuda.get_device_properties(0).multi_processor_count


def traffic_for(workload: str, source: str):
    """HBM bytes per launch of the kernel built from KERNEL_SOURCES[source] on this
    workload, from committed rocprofv3 counters, or None.

    None when no counters were taken for this workload and kernel, or when the
    kernel's source or compile flags changed since they were (their hash is stored
    next to them).
    """
    try:
        with open(TRAFFIC_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    entry = table.get(workload, {}).get(source)
    if not entry or entry.get("kernel_source_sha256") != kernel_hash(source):
        return None
    return entry.get("traffic_bytes_per_launch")


def counters_for(workload: str, source: str):
    """Shader counters of the kernel built from KERNEL_SOURCES[source] (or of one kernel of it,
    "source/part") on this workload, from
    a committed rocprofv3 pass: the kernel's own shader clock, MFMA busy share at that clock,
    LDS activity and bank conflicts.  None when absent or when the kernel changed since."""
    try:
        with open(SQ_FILE) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    entry = table.get(workload, {}).get(source)   # "bwd/dq": one kernel of a multi-kernel source
    if not entry or entry.get("kernel_source_sha256") != kernel_hash(source.split("/")[0]):
        return None
    keys = ("sclk_ghz", "mfma_busy", "mfma_insts_over_algorithmic", "valu_insts_per_mfma",
            "lds_insts_per_mfma", "lds_idx_active", "lds_bank_conflict_rate", "kernel_us_under_counters")
    out = {k: entry[k] for k in keys if k in entry}
    out["source"] = "a committed rocprofv3 --pmc pass of the same kernel (profiles/sq_counters.json), not this run"
    return out


def precondition(call, seconds):
    """Run ``call`` back to back for about ``seconds`` of wall time (batches of 8 launches
    between synchronisations), so that the timed steps see the clock the GPU holds under
    sustained load rather than its ramp.  Returns what was done."""
    import torch

    if seconds <= 0:
        return {"seconds": 0.0, "launches": 0}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            call()
        n += 8
        torch.cuda.synchronize()
    return {"seconds": time.perf_counter() - t0, "launches": n,
            "why": "the GPU raises its clock over the first tens of ms of sustained MFMA work"}


def stamped_clock(w, q, k, v, o, lse):
    """Shader clock of one launch, from the kernel's per-wave counters: the ratio of
    shader cycles to real-time ticks over every wave, times the real-time counter's rate.
    One launch is stamped twice (the second is reported) right after the timed loop."""
    import torch

    from flashattention_online_softmax_fwd_amd import _lib

    code = {"bf16": _lib.FA_DTYPE_BF16, "f16": _lib.FA_DTYPE_F16}.get(w.dtype)
    if code is None:
        return None
    slots = _lib.fa_fwd_stamp_slots(w.B, w.Hq, w.N, w.d, code)
    khz = _lib.fa_wall_clock_khz(q.device.index or 0)
    simds = 4 * torch.cuda.get_device_properties(q.device).multi_processor_count
    if slots <= 0 or khz <= 0:
        return None
    stamps = torch.zeros(slots * 4, dtype=torch.int64, device=q.device)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        rc = _lib.fa_fwd_stamped(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 w.B, w.Hq, w.Hkv, w.N, w.d, int(w.causal), w.softmax_scale, code,
                                 stream.cuda_stream, stamps.data_ptr(), slots)
        if rc != 0:
            raise RuntimeError("fa_fwd_stamped: " + _lib.fa_last_error())
    torch.cuda.synchronize()
    st = stamps.view(slots, 4).cpu().numpy().astype("int64")
    st = st[st[:, 1] != 0]                 # slots past the launch's waves stay zero
    real = st[:, 1] - st[:, 0]
    cyc = st[:, 3] - st[:, 2]
    span_ticks = int(st[:, 1].max() - st[:, 0].min())
    return {
        "sclk_ghz": float(cyc.sum()) / float(real.sum()) * khz * 1e3 / 1e9,
        "kernel_span_ms": span_ticks / khz,
        "waves": int(len(st)),
        # share of SIMD time the waves held: the 16-bit kernels run one wave per SIMD
        "simd_busy": float(real.sum()) / float(span_ticks * simds) if simds else None,
        "wave_ms_mean": float(real.mean()) / khz,
        "wave_ms_max": float(real.max()) / khz,
        "wall_clock_khz": khz,
        "source": "fa_fwd_stamped: s_memtime / s_memrealtime per wave, one launch after the timed loop",
    }


def time_gpu(fa, q, k, v, w, steps, warmup, precondition_s):
    import torch

    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=q.device)

    def call():
        fa.forward(q, k, v, causal=w.causal, scale=w.softmax_scale, out=o, lse=lse)

    pre = precondition(call, precondition_s)
    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, per_launch_ms, o, lse, pre


def cpu_baseline(w, q, k, v, o, lse, budget_s):
    """Time the fp64 oracle on seeded sample rows until about budget_s seconds."""
    import numpy as np

    from flashattention_online_softmax_fwd_amd import inputs as fin
    from oracle import fa_oracle

    total = w.B * w.Hq * w.N
    order = fin.sample_rows(w, total if total <= 1 << 20 else 1 << 20, seed=w.seed + 7)
    np.random.default_rng(w.seed + 8).shuffle(order)
    qh, kh, vh = (fa_oracle._as_f64(t) for t in (q, k, v))   # exact upcast, outside the timing
    done, spent, chunk = [], 0.0, 64
    outs, lses = [], []
    pos = 0
    while spent < budget_s and pos < len(order):
        rows = np.sort(order[pos:pos + chunk])
        pos += len(rows)
        t0 = time.perf_counter()
        ro, rl = fa_oracle.attention(qh, kh, vh, causal=w.causal, scale=w.softmax_scale, rows=rows)
        spent += time.perf_counter() - t0
        done.append(rows)
        outs.append(ro)
        lses.append(rl)
        chunk = min(chunk * 2, 4096)
    rows = np.concatenate(done)
    ro = np.concatenate(outs)
    rl = np.concatenate(lses)
    flops = fa_oracle.row_flops(w.N, w.d, w.causal, rows)
    go = o.reshape(-1, w.d)[torch_index(rows, o.device)].float().cpu().numpy()
    gl = lse.reshape(-1)[torch_index(rows, o.device)].cpu().numpy()
    from oracle import tolerances
    ok = tolerances.within(go, ro, w.dtype) and tolerances.within(gl, rl, w.dtype)
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": fa_oracle.num_threads(),
        "kind": "oracle",
        "sample": "%d seeded query rows of %s (%.3g of its %.3g flops), fp64 three-pass oracle, %.1f s"
                  % (len(rows), w.name, flops, w.flops, spent),
        "seconds": spent,
        "rows": int(len(rows)),
        # the whole workload on the oracle: measured when the sample is every row, else the
        # sample's time scaled by the workload's flops over the sample's
        "full_problem_seconds": spent * w.flops / flops,
        "full_problem_seconds_kind": "measured" if len(rows) == total else "extrapolated",
        "gpu_matches_oracle_on_sample": ok,
        "max_abs_err_o": float(np.abs(go - ro).max()),
        "max_abs_err_lse": float(np.abs(gl - rl).max()),
    }


def torch_index(rows, device):
    import torch
    return torch.as_tensor(rows, dtype=torch.long, device=device)


def run_workload(name, steps, warmup, with_cpu, cpu_budget, precondition_s=0.0):
    import torch

    import flashattention_online_softmax_fwd_amd as fa
    from flashattention_online_softmax_fwd_amd import inputs as fin

    fa.load_library()
    w = fin.WORKLOADS[name]
    q, k, v = fin.workload_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    torch.cuda.synchronize()
    src, kname = forward_kernel(w, device_simds())
    wall, per_ms, o, lse, pre = time_gpu(fa, qd, kd, vd, w, steps, warmup, precondition_s)
    clock = stamped_clock(w, qd, kd, vd, o, lse)
    if clock and src != "w64":
        clock["simd_busy"] = None        # the 32-rows-per-wave kernel runs two waves per SIMD
    ms_step = wall * 1e3 / steps
    tflops = w.flops * steps / wall / 1e12
    avg_launch_ms = sum(per_ms) / len(per_ms)
    achieved = w.flops / (avg_launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    rec = {
        "metric": metric_for(w),
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal Q/K/V, numpy default_rng(%d)%s)"
                % (w.seed, ", Q x %g" % w.q_mult if w.q_mult != 1.0 else ""),
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "scale": w.softmax_scale, "dtype": w.dtype,
                   "flops_per_step": w.flops},
        "frac_of_peak": tflops / peak,
        "hbm_gbps": w.algorithmic_bytes / (avg_launch_ms * 1e-3) / 1e9,
        # for contrast only: one fp32 write of the N x N score table per head, which the
        # tiled method never makes (the textbook path also reads it back at least once)
        "textbook_score_bytes": 4 * w.B * w.Hq * w.N * w.N,
        "roofline": {
            "bound": "mfma",
            "achieved": achieved,
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": achieved / peak,
            "traffic": traffic_for(w.name, src),
            "kernel": kname,
            "avg_launch_ms": avg_launch_ms,
            "min_launch_ms": min(per_ms),
            "median_launch_ms": sorted(per_ms)[len(per_ms) // 2],
            "launch_ms_first5": per_ms[:5],
            "launch_ms_last5": per_ms[-5:],
            "algorithmic_flops_per_launch": w.flops,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes,
        },
        "preconditioning": pre,
        "clock": clock,
        "counters": counters_for(w.name, src),
    }
    if with_cpu:
        rec["cpu_baseline"] = cpu_baseline(w, q, k, v, o, lse, cpu_budget)
    return rec


def run_kv_workload(name, steps, warmup):
    """Split-KV + merge over a decode-shaped workload: one step is both launches.

    Reading the K/V cache dominates, so each kernel is priced against HBM: its
    algorithmic bytes (what it must read and write at least once) over its
    average launch duration from HIP events on the launch stream.
    """
    import torch

    import flashattention_online_softmax_fwd_amd as fa
    from flashattention_online_softmax_fwd_amd import _lib
    from flashattention_online_softmax_fwd_amd import inputs as fin

    fa.load_library()
    w = fin.KV_WORKLOADS[name]
    q, k, v = fin.kv_workload_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    S = _lib.fa_splitkv_num_splits(w.B, w.Hq, w.Hkv, w.Nq, w.Nk)
    rows = w.B * w.Hq * w.Nq
    o_part = torch.empty((S, w.B, w.Hq, w.Nq, w.d), dtype=torch.float32, device=dev)
    lse_part = torch.empty((S, w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def split():
        rc = _lib.fa_fwd_splitkv(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_part.data_ptr(),
                                 lse_part.data_ptr(), w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d, int(w.causal),
                                 w.softmax_scale, _lib.FA_DTYPE_BF16, S, sh)
        assert rc == 0, _lib.fa_last_error()

    def merge():
        rc = _lib.fa_merge(o_part.data_ptr(), lse_part.data_ptr(), o.data_ptr(), lse.data_ptr(), S, w.B,
                           w.Hq, w.Nq, w.d, _lib.FA_DTYPE_BF16, sh)
        assert rc == 0, _lib.fa_last_error()

    for _ in range(warmup):
        split()
        merge()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        split()
        ev[i][1].record(stream)
        merge()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    split_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    merge_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    part_bytes = S * rows * (w.d + 1) * 4
    split_bytes = 2 * w.B * w.d * (w.Hq * w.Nq + 2 * w.Hkv * w.Nk) + part_bytes
    merge_bytes = part_bytes + rows * (2 * w.d + 4)

    def roof(kernel, source, nbytes, ms):
        gbps = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": gbps / PEAK_HBM_GBPS, "traffic": traffic_for(w.name, source), "kernel": kernel,
                "avg_launch_ms": ms, "algorithmic_bytes_per_launch": nbytes}

    return {
        "metric": "split-KV attention (split + merge) effective HBM GB/s",
        "value": w.algorithmic_bytes * steps / wall / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": wall * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal Q/K/V, numpy default_rng(%d))" % w.seed,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Nq": w.Nq, "Nk": w.Nk,
                   "d": w.d, "causal": w.causal, "num_splits": S, "flops_per_step": w.flops,
                   "algorithmic_bytes_per_step": w.algorithmic_bytes},
        "tflops": w.flops * steps / wall / 1e12,
        "roofline": roof("fa::fwd16_kernel<bf16, split>", "bf16", split_bytes, split_ms),
        "merge_roofline": roof("fa::merge_kernel", "merge", merge_bytes, merge_ms),
    }


# Reads and writes per element of each row-softmax algorithm (spicyshark.co lesson, "The cost:
# three passes" and "Why reading once matters").
SOFTMAX_ACCESSES = {"online": (2, 1), "safe": (3, 1)}
ROW_ON_CHIP_BYTES = 64 * 1024   # a row this long fits in one workgroup's share of a CU's 160 KB LDS


def run_softmax_workload(name, steps, warmup):
    """Row softmax of a [rows, cols] matrix by both algorithms; one step is one launch.

    Each algorithm is priced against HBM with its own access count (the bytes it
    must move when a row is too long to stay on chip between its passes; a row that
    fits in one workgroup's LDS is priced at x once and y once); ``value`` is the
    online algorithm's effective rate, x read once plus y written once, over its
    wall time.
    """
    import torch

    import flashattention_online_softmax_fwd_amd as fa
    from flashattention_online_softmax_fwd_amd import _lib
    from flashattention_online_softmax_fwd_amd import inputs as fin

    fa.load_library()
    w = fin.SOFTMAX_WORKLOADS[name]
    dev = torch.device("cuda:0")
    x = fin.softmax_workload_inputs(w).to(dev)
    y = torch.empty_like(x)
    lse = torch.empty((w.rows,), dtype=torch.float32, device=dev)
    dt = {"f32": _lib.FA_DTYPE_F32, "bf16": _lib.FA_DTYPE_BF16, "f16": _lib.FA_DTYPE_F16}[w.dtype]
    stream = torch.cuda.current_stream()
    out = {}
    for algo, code in (("online", _lib.FA_SOFTMAX_ONLINE), ("safe", _lib.FA_SOFTMAX_SAFE)):
        def call():
            rc = _lib.fa_softmax(x.data_ptr(), y.data_ptr(), lse.data_ptr(), w.rows, w.cols, dt, code,
                                 stream.cuda_stream)
            assert rc == 0, _lib.fa_last_error()
        for _ in range(warmup):
            call()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for a, b in ev:
            a.record(stream)
            call()
            b.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = sum(a.elapsed_time(b) for a, b in ev) / steps
        reads, writes = SOFTMAX_ACCESSES[algo]
        # A row that fits in one workgroup's LDS could be read from HBM once whatever the
        # algorithm, so only x once and y once are algorithmic; a longer row must be read
        # from HBM as often as the algorithm passes over it.
        if w.cols * w.esize <= ROW_ON_CHIP_BYTES:
            reads, writes = 1, 1
        nbytes = (reads + writes) * w.rows * w.cols * w.esize + 4 * w.rows
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[algo] = {"wall_s": wall, "ms": ms, "roofline": {
            "bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
            "traffic": traffic_for(w.name + ":" + algo, "softmax"), "kernel": "fa::softmax_kernel (%s)" % algo,
            "avg_launch_ms": ms, "algorithmic_bytes_per_launch": nbytes,
            "accesses_per_element": reads + writes}}
    on, sa = out["online"], out["safe"]
    return {
        "metric": "row softmax effective GB/s (x read once, y written once), online algorithm",
        "value": w.io_bytes * steps / on["wall_s"] / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": on["wall_s"] * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal scores x %g, numpy default_rng(%d))" % (w.sigma, w.seed),
        "config": {"workload": w.name, "rows": w.rows, "cols": w.cols, "dtype": w.dtype,
                   "io_bytes_per_step": w.io_bytes},
        "roofline": on["roofline"],
        "safe_roofline": sa["roofline"],
        "online_speedup_over_safe": sa["ms"] / on["ms"],
    }


def run_bwd_workload(name, steps, warmup):
    """Backward pass (dq, dk, dv from q, k, v, o, lse and dO); one step is one fa_bwd_split
    call with fa_bwd_num_splits splits: its kernels (dq with D = rowsum(dO o), dk/dv, and
    the sum of the dk/dv partials when there are several splits) back to back on one stream.

    ``value`` counts the five products of the backward (S, dP, dV, dK, dQ: 2.5 times
    the forward's flops) per step over the timed wall time.  The kernels recompute S
    and dP once more (in the dq kernel and in the dk/dv kernel), which the count
    leaves out.  ``roofline`` prices the call's average duration, from HIP events on
    its stream, against the dense bf16 MFMA peak; the per-kernel split is in the
    rocprofv3 summary.
    """
    import torch

    import flashattention_online_softmax_fwd_amd as fa
    from flashattention_online_softmax_fwd_amd import _lib
    from flashattention_online_softmax_fwd_amd import inputs as fin

    fa.load_library()
    w = fin.BWD_WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v, do = (t.to(dev) for t in fin.bwd_workload_inputs(w))
    o, lse = fa.forward(q, k, v, causal=w.causal, scale=w.softmax_scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((w.B, w.Hq, w.N), dtype=torch.float32, device=dev)
    S = _lib.fa_bwd_num_splits(w.B, w.Hq, w.Hkv, w.N)
    part = torch.empty((2, S) + tuple(k.shape), dtype=torch.float32, device=dev) if S > 1 else None
    dt = {"bf16": _lib.FA_DTYPE_BF16, "f16": _lib.FA_DTYPE_F16}[w.dtype]
    stream = torch.cuda.current_stream()

    def call():
        rc = _lib.fa_bwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                               part.data_ptr() if part is not None else None, S, w.B, w.Hq, w.Hkv, w.N, w.d,
                               int(w.causal), w.softmax_scale, dt, stream.cuda_stream)
        assert rc == 0, _lib.fa_last_error()

    for _ in range(warmup):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    flops = fin.bwd_flops(w)
    achieved = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    return {
        "metric": "attention bwd TFLOP/s (5 products, 2.5x the forward's flops)",
        "value": flops * steps / wall / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": wall * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded normal Q/K/V/dO, numpy default_rng(%d), dO seed + 50000)" % w.seed,
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "d": w.d,
                   "causal": w.causal, "dkdv_splits": S, "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic_for(w.name, "bwd"),
                     "kernel": "fa_bwd_split (fa::bwd_dq_kernel + fa::bwd_dkdv_kernel [+ fa::bwd_reduce_kernel])",
                     "avg_launch_ms": ms, "algorithmic_flops_per_launch": flops},
        "counters": {part: counters_for(w.name, "bwd/" + part) for part in ("dq", "dkdv")},
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU clock ramps up over the first tens of milliseconds of sustained MFMA work,
    # so the default warm-up is long enough (~65 ms at the default workload) to reach it.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=None,
                    help="one of inputs.WORKLOADS, KV_WORKLOADS, SOFTMAX_WORKLOADS or BWD_WORKLOADS "
                         "(default: the metric's)")
    ap.add_argument("--all", action="store_true", help="one line per workload (no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--precondition-seconds", type=float, default=0.3,
                    help="run the kernel back to back this long before the warm-up steps (0: off)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, run torch.neg over 256 MiB of float32 three times: a plain "
                         "kernel that reads and writes known byte counts, for scaling HBM counters")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU and has no multi-GPU path: run it with --gpus 1", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 2
    from flashattention_online_softmax_fwd_amd import inputs as fin
    if args.all:
        for name in fin.WORKLOADS:
            print(json.dumps(run_workload(name, args.steps, args.warmup, False, 0.0, args.precondition_seconds)),
                  flush=True)
        for name in fin.KV_WORKLOADS:
            print(json.dumps(run_kv_workload(name, args.steps, args.warmup)), flush=True)
        for name in fin.SOFTMAX_WORKLOADS:
            print(json.dumps(run_softmax_workload(name, args.steps, args.warmup)), flush=True)
        for name in fin.BWD_WORKLOADS:
            print(json.dumps(run_bwd_workload(name, args.steps, args.warmup)), flush=True)
        return 0
    name = args.workload or fin.BENCH_WORKLOAD
    if name in fin.KV_WORKLOADS:
        rec = run_kv_workload(name, args.steps, args.warmup)
    elif name in fin.SOFTMAX_WORKLOADS:
        rec = run_softmax_workload(name, args.steps, args.warmup)
    elif name in fin.BWD_WORKLOADS:
        rec = run_bwd_workload(name, args.steps, args.warmup)
    else:
        rec = run_workload(name, args.steps, args.warmup, not args.no_cpu_baseline, args.cpu_seconds,
                           args.precondition_seconds)
    if args.copy_calibration:
        x = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.neg(x, out=y)
        torch.cuda.synchronize()
        rec["copy_calibration"] = {"kernel": "torch.neg float32", "read_bytes": x.numel() * 4,
                                   "write_bytes": y.numel() * 4, "launches": 3}
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
