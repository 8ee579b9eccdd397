#!/usr/bin/env python
"""Throughput of the SSD chunked-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one full forward over one batch of seeded synthetic inputs
already resident in HBM: y with the D skip, the final state, and the state
at the accepted index where the workload asks for it.  The headline workload
is the Mamba-2 2.7B layer shape (b=8, T=2048, H=80, P=64, N=128, G=1, Q=256,
bf16 in, fp32 state, zero initial state); the other four workloads are timed
too and reported under "workloads".  Prints ONE JSON line.

Timing has one source: HIP events recorded on the stream the library's
kernels run on (torch's current stream, which the binding passes down).
"value" and "ms_per_step" are the K steps back to back between the first
and the last event (warm: whatever the 256 MB last-level cache keeps between
steps); events also close each of up to 10 groups of those steps, whose means
give the warm median and min (an event between every two steps would add its
own gap to each).  The cold figures time single steps, each after a 512 MiB
buffer is written on the same stream, which evicts the caches.

The roofline entry is for the dominant kernel.  On the automatic path the
headline step is ONE kernel (the single pass), so its average launch
duration is the warm mean per step.  Its algorithmic bytes are the step's
minimal HBM traffic: x and y, B and C, dt, the final state (and the initial
state / state at index where present), each once.  Measured HBM traffic
comes from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/
when that was taken on the current kernel source (else null).

Other modes:
    --copy-probe          also run a plain 256 MiB device copy (counter calibration)
    --path P              time a given path (auto, one_chunk, single_pass, chunk_parallel)
    --summarize-pmc D...  turn rocprofv3 --pmc output dirs into profiles/ summaries
    --summarize-stats D   turn a rocprofv3 --kernel-trace --stats dir into a profiles/ summary
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ssd_inputs  # noqa: E402

METRIC = "SSD fwd tokens/s and TFLOP/s (% of MI355X bf16 MFMA peak), 2.7B-layer shape"
HEADLINE = "mamba2_2.7b"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (vector and MFMA)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SOURCES = {
    "chunk_cumsum": ["chunk_cumsum.hip"],
    "chunk_state": ["chunk_state_heads.hip", "chunk_state.hip", "device_common.hpp"],
    "state_pass": ["state_pass.hip", "device_common.hpp"],
    "chunk_output": ["chunk_output_heads.hip", "chunk_output.hip", "device_common.hpp"],
    "chunk_scan_fused": ["chunk_scan_fused.hip", "device_common.hpp"],
    "one_chunk": ["one_chunk.hip", "device_common.hpp"],
    "empty_sequence": ["state_pass.hip"],
    "state_correction": ["state_correction.hip", "device_common.hpp"],
}
# One GPU's shard of the 16K-token dstate-256 workload on 8 GPUs (2048 tokens),
# corrected in place once the state entering it is known (sequence sharding).
CP_SHARD = ssd_inputs.Workload("long_16k_n256_shard", 1, 2048, 64, 64, 256, 1, 256, "bf16", init_state=True,
                               seed=1102)
ALL_WORKLOADS = {**ssd_inputs.WORKLOADS, CP_SHARD.name: CP_SHARD}
CSRC = os.path.join(ROOT, "mamba_ssd_scan_06_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# ------------------------------------------------------------ work per kernel
def chunk_lengths(wl):
    Q, T = wl.chunk, wl.seqlen
    return [min(Q, T - c) for c in range(0, T, Q)]


def step_bytes(wl):
    """Minimal HBM bytes of one step: every input read once and every output
    written once (x, y, B, C, dt, the final state, and the initial state and
    the state at the accepted index where the workload has them)."""
    b, T, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    e = 2 if wl.dtype == "bf16" else 4
    st = b * H * P * N * 4
    return (2 * b * T * H * P * e + 2 * b * T * G * N * e + b * T * H * 4 + 2 * H * 4 + st
            + (st if wl.init_state else 0) + (st + 4 * b if wl.state_out else 0))


def correction_bytes(wl):
    """Minimal HBM bytes of ssd_state_correction on a shard: y read and
    written, C, dt and A read, h_in and the shard's final state read, the
    corrected final state written."""
    b, T, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    e = 2 if wl.dtype == "bf16" else 4
    return 2 * b * T * H * P * e + b * T * G * N * e + b * T * H * 4 + H * 4 + 3 * b * H * P * N * 4


def kernel_bytes(wl):
    """Minimal HBM bytes of each chunk-parallel kernel on its own: the
    tensors it must read or write once, including the workspace
    intermediates it exchanges with the other kernels (cs, ct, dte in fp32,
    the chunk states and the states entering each chunk in the input
    dtype).  The single pass and one_chunk exchange nothing: their bytes are
    the step's."""
    b, T, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    e = 2 if wl.dtype == "bf16" else 4
    nc = len(chunk_lengths(wl))
    x, bc, dt = b * T * H * P * e, b * T * G * N * e, b * T * H * 4
    tab = b * H * nc * wl.chunk * 4
    st = b * H * P * N * 4
    S = nc * st // 4 * e
    prev = (nc if wl.init_state else nc - 1) * st // 4 * e
    out = {"chunk_cumsum": dt + 3 * tab,
           "chunk_state": x + bc + dt + tab + S,
           "state_pass": S + prev + st + (st if wl.init_state else 0),
           "chunk_output": 2 * x + 2 * bc + 3 * tab + prev,
           "chunk_scan_fused": step_bytes(wl), "one_chunk": step_bytes(wl),
           "state_correction": correction_bytes(wl)}
    return out


def total_flops(wl):
    """Algorithmic flops of one step of the block decomposition at the
    workload's chunk size: per chunk of q tokens, C.B^T over the causal
    triangle once per group, the masked product with x per head, the chunk
    state and the state-to-output product per head."""
    qs = chunk_lengths(wl)
    b, H, P, N, G = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    return b * sum(G * q * (q + 1) * N + H * q * (q + 1) * P + 4 * H * q * N * P for q in qs)


def kernel_flops(wl):
    """Algorithmic flops of each kernel that contracts on the matrix cores
    (the causal triangle counted once; C.B^T once per chunk and group)."""
    qs = chunk_lengths(wl)
    b, H, P, N, G = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    prior = sum(qs[1:]) + (qs[0] if wl.init_state and qs else 0)
    return {"chunk_state": 2 * b * H * N * P * wl.seqlen,
            "chunk_output": b * sum(G * q * (q + 1) * N + H * q * (q + 1) * P for q in qs) + 2 * b * H * N * P * prior,
            "chunk_scan_fused": total_flops(wl), "one_chunk": total_flops(wl),
            "state_correction": 2 * b * H * N * P * wl.seqlen}


def timed_mean_us(key, workload):
    """A kernel's mean duration in the kernel-trace summary of the same
    workload (the timed steps where the summary has them, else all calls)."""
    path = os.path.join(PROFILES, f"kernels_{workload}_kernel_stats.txt")
    if not os.path.exists(path):
        return None
    timed, calls = None, None
    with open(path) as f:
        for line in f:
            parts = [x.strip() for x in line.split("|")]
            if line.startswith("timed |") and len(parts) >= 4 and _kernel_key(parts[1]) == key:
                timed = float(parts[3]) / 1e3
            elif not line.startswith("#") and len(parts) >= 4 and _kernel_key(parts[0]) == key:
                calls = float(parts[3]) / 1e3
    return timed if timed is not None else calls


def source_hash(kernel):
    """Hash of a kernel's sources and of the compiler flags they are built
    with (absolute include paths left out, so the hash is the same in every
    checkout)."""
    from mamba_ssd_scan_06_amd import build as _build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
        flags = [a for a in _build.HIPCC_FLAGS + _build.EXTRA_FLAGS.get(f, []) if not os.path.isabs(a)]
        h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ running
def device_inputs(inp, device):
    import numpy as np
    import torch

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)

    if inp.wl.dtype == "bf16":
        x, B, C = bf16(inp.x_bits), bf16(inp.B_bits), bf16(inp.C_bits)
    else:
        x, B, C = (torch.from_numpy(getattr(inp, k)).to(device) for k in ("x", "B", "C"))
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(x=x, dt=t(inp.dt), A=t(inp.A), B=B, C=C, D=t(inp.D), init_state=t(inp.init_state),
                state_out_idx=t(inp.state_out_idx))


def _stats(us, n_steps=None):
    s = sorted(us)
    return {"mean_us": round(sum(s) / len(s), 2), "median_us": round(s[len(s) // 2], 2), "min_us": round(s[0], 2),
            "max_us": round(s[-1], 2), "samples": len(s), "steps": n_steps or len(s)}


FLUSH_BYTES = 512 << 20


def time_workload(wl, steps, warmup, device, path_name="auto", cold_steps=10):
    """Times `steps` forwards of `wl` back to back (warm) and `cold_steps`
    single forwards after a cache flush.  Returns (inputs, result dict)."""
    import torch

    import mamba_ssd_scan_06_amd as ssd

    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp, device)
    b, T, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    code = ssd.SSD_DTYPE_BF16 if wl.dtype == "bf16" else ssd.SSD_DTYPE_F32
    shape = ssd.make_shape(b, T, H, P, N, G)
    path = {v: k for k, v in ssd.PATH_NAMES.items()}[path_name]
    run_path = path if path != ssd.SSD_PATH_AUTO else ssd.ssd_select_path(shape, wl.chunk, code)
    ws_bytes = ssd.ssd_get_workspace_layout(shape, wl.chunk, code).total_bytes \
        if run_path == ssd.SSD_PATH_CHUNK_PARALLEL else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device) if ws_bytes else None
    y = torch.empty_like(dev["x"])
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device=device)
    sout = torch.empty_like(fin) if wl.state_out else None
    args = (dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["init_state"], wl.chunk,
            dev["state_out_idx"])
    kw = dict(y=y, final_state=fin, state_out=sout, workspace=ws, path=path)
    # The kernels one step launches (one untimed call with marks).
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
    for m in marks:
        m.record()
    *_, names = ssd.ssd_chunk_scan_fwd_ex(*args, marks=[m.cuda_event for m in marks], **kw)
    for _ in range(warmup):
        ssd.ssd_chunk_scan_fwd_ex(*args, **kw)
    torch.cuda.synchronize()
    # Warm: K steps back to back in `blocks` groups, an event before the first
    # step and after each group (an event between every two steps would add
    # its own gap to each); the median and min are over the groups' means.
    blocks = max(1, min(10, steps // 10))
    bounds = [steps * g // blocks for g in range(blocks + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
    t0 = time.perf_counter()
    evs[0].record()
    for g in range(blocks):
        for _ in range(bounds[g], bounds[g + 1]):
            ssd.ssd_chunk_scan_fwd_ex(*args, **kw)
        evs[g + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm_us = [evs[g].elapsed_time(evs[g + 1]) * 1e3 / (bounds[g + 1] - bounds[g]) for g in range(blocks)]
    ms_step = evs[0].elapsed_time(evs[blocks]) / steps
    # Cold: each step after 512 MiB are written on the same stream.
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=device)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(cold_steps)]
    for k, (e0, e1) in enumerate(pairs):
        flush.fill_(float(k))
        e0.record()
        ssd.ssd_chunk_scan_fwd_ex(*args, **kw)
        e1.record()
    torch.cuda.synchronize()
    cold_us = [e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs]
    del flush
    warm = dict(_stats(warm_us, steps), mean_us=round(ms_step * 1e3, 2))
    return inp, dict(ms_per_step=ms_step, wall_s=wall, warm=warm, cold=_stats(cold_us),
                     kernels=names, path=ssd.PATH_NAMES[run_path])


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from profiles/<kernel>_<workload>_counters.txt, if
    the counters were taken on the current kernel source."""
    vals = read_profile(kernel, workload)
    if vals is None or vals.get("kernel_source_sha256") != source_hash(kernel):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def read_profile(kernel, workload):
    path = os.path.join(PROFILES, f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    return vals


def roofline_entry(wl, res):
    """Roofline of the dominant kernel.  A one-kernel step's kernel is timed
    by the step's events; for a step of several kernels the entry covers the
    whole step (named as such)."""
    ms = res["ms_per_step"]
    names = res["kernels"]
    kernel = names[0] if len(names) == 1 else "step (" + " + ".join(names) + ")"
    alg_bytes = step_bytes(wl)
    flops = total_flops(wl)
    peak_flops = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    ai = flops / alg_bytes
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    traffic = traffic_from_profile(names[0], wl.name) if len(names) == 1 else None
    common = {"kernel": kernel, "traffic": traffic, "alg_bytes": alg_bytes, "alg_flops": flops,
              "avg_launch_us": round(ms * 1e3, 2), "arith_intensity": round(ai, 1), "ridge": round(ridge, 1)}
    if ai >= ridge:
        achieved = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_flops, "unit": "TFLOP/s",
                "frac": round(achieved / peak_flops, 4), **common}
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), **common}


# Single-token decode at the 2.7B-layer shape: the state updated in place.
DECODE = ssd_inputs.Workload("decode_2.7b_b256", 256, 1, 80, 64, 128, 1, 256, "bf16", init_state=True, seed=1101)


def time_decode(steps, warmup, device):
    """One-token calls with final_state = init_state (in place), back to back."""
    import torch

    import mamba_ssd_scan_06_amd as ssd

    wl = DECODE
    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp, device)
    h = dev["init_state"]
    y = torch.empty_like(dev["x"])
    args = (dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], h, wl.chunk)
    for _ in range(warmup):
        ssd.ssd_chunk_scan_fwd(*args, y=y, final_state=h)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        ssd.ssd_chunk_scan_fwd(*args, y=y, final_state=h)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    b, H, P, N = wl.batch, wl.nheads, wl.headdim, wl.dstate
    state_bytes = 2 * b * H * P * N * 4  # read and write the fp32 state
    return {"workload": wl.name, "batch": b, "nheads": H, "headdim": P, "dstate": N, "in_place": True,
            "us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(b / (ms * 1e-3), 1),
            "state_GB/s": round(state_bytes / (ms * 1e-3) / 1e9, 1)}


def time_state_correction(steps, warmup, device):
    """ssd_state_correction on a sequence shard, back to back on the same
    buffers (each call adds the correction again: the values change, the
    work does not), next to the shard's own forward from a zero state."""
    import torch

    import mamba_ssd_scan_06_amd as ssd

    wl = CP_SHARD
    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp, device)
    b, T, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    y, fin, _ = ssd.ssd_chunk_scan_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], None, wl.chunk)
    h_in = dev["init_state"]
    out = torch.empty_like(fin)

    # The binding checks every tensor on each call, which takes longer than
    # the kernel: the timed loop calls the C entry point with its arguments
    # marshalled once (the first call goes through the binding's checks).
    ssd.ssd_state_correction(y, dev["dt"], dev["A"], dev["C"], h_in, shard_final=fin, final_state=out)
    lib = ssd._load()
    shape = ssd.make_shape(b, T, H, P, N, G)
    stream = ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)
    cargs = (ssd._ptr(y), ssd._ptr(dev["dt"]), ssd._ptr(dev["A"]), ssd._ptr(dev["C"]), ssd._ptr(h_in),
             ssd._ptr(fin), ssd._ptr(out), None, None, ctypes.byref(shape), ssd.SSD_DTYPE_BF16, stream)

    def corr():
        if lib.ssd_state_correction(*cargs) != 0:
            raise RuntimeError(ssd.ssd_last_error())

    def fwd():
        ssd.ssd_chunk_scan_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], None, wl.chunk,
                               y=y, final_state=fin)

    def timed(f):
        for _ in range(warmup):
            f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    us = timed(corr)
    fwd_us = timed(fwd)
    nbytes = correction_bytes(wl)
    return {"workload": wl.name, "batch": b, "seqlen": T, "nheads": H, "headdim": P, "dstate": N,
            "us_per_call": round(us, 2), "alg_bytes": nbytes, "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(nbytes / (us * 1e-6) / (PEAK_HBM_GBS * 1e9), 4),
            "shard_forward_us": round(fwd_us, 2)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, inp, seqs=None):
    """The fp64 oracle on the host cores, on the first `seqs` sequences of the
    workload (all heads, all tokens; default all of them): once on one
    thread, once on every core this process may use."""
    import oracle

    cores = len(os.sched_getaffinity(0))
    n = min(seqs or wl.batch, wl.batch)
    sl = lambda a: None if a is None else a[:n]
    sample = (sl(inp.x), sl(inp.dt), inp.A, sl(inp.B), sl(inp.C), inp.D, sl(inp.init_state), sl(inp.state_out_idx))
    tokens = n * wl.seqlen
    runs = {}
    for threads in (1, cores):
        t0 = time.perf_counter()
        oracle.ssd_forward(*sample, nthreads=threads)
        runs[threads] = time.perf_counter() - t0
    return {"value": round(tokens / runs[cores], 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the first {n} of {wl.batch} sequences of {wl.name} ({tokens} tokens, all {wl.nheads} "
                      f"heads), fp64 recurrence, one pass: {runs[cores]:.2f} s on {cores} threads, "
                      f"{runs[1]:.2f} s on 1",
            "one_core": {"value": round(tokens / runs[1], 1), "unit": "tokens/s", "cores": 1},
            "cpu_model": cpu_model()}


def copy_probe(device):
    """A plain device-to-device copy of 256 MiB (counter calibration for --pmc runs)."""
    import torch

    n = 256 << 20
    src = torch.ones(n // 4, dtype=torch.float32, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


# ------------------------------------------------------------ profile summaries
def _read_csv(pattern):
    files = glob.glob(pattern, recursive=True)
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return files, rows


def summarize_stats(d, workload=HEADLINE, command="", steps=None, warmup=None, cold_steps=None):
    """The rocprofv3 kernel statistics of a bench.py run, and for each kernel
    launched once per step, its mean and median duration over the timed
    steps alone (bench.py launches one marked step, then `warmup` steps,
    then the `steps` timed ones, then `cold_steps` after cache flushes)."""
    files, rows = _read_csv(os.path.join(d, "**", "*kernel_stats.csv"))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    lines = [f"# rocprofv3 kernel-trace statistics, workload {workload}", f"# command: {command}",
             "# name | calls | total_ns | avg_ns | min_ns | max_ns | pct"]
    for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
        name = r.get("Name", "")
        short = (name[:name.rfind("(")] if name.endswith(")") else name)[-90:]
        lines.append(f"{short} | {r.get('Calls')} | {r.get('TotalDurationNs')} | {float(r.get('AverageNs', 0)):.0f} | "
                     f"{r.get('MinNs')} | {r.get('MaxNs')} | {float(r.get('Percentage', 0)):.2f}")
    _, trace = _read_csv(os.path.join(d, "**", "*kernel_trace.csv"))
    if trace and steps is not None and warmup is not None:
        per = {}
        for r in trace:
            per.setdefault(r["Kernel_Name"], []).append(
                (int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        n_expected = 1 + warmup + steps + (cold_steps or 0)
        lines.append(f"# timed steps only (dispatches {1 + warmup} .. {warmup + steps} of each step kernel, "
                     f"in launch order): name | steps | mean_ns | median_ns")
        for name, ds in per.items():
            if len(ds) != n_expected:
                continue
            ds.sort()
            t = sorted(v for _, v in ds[1 + warmup:1 + warmup + steps])
            short = (name[:name.rfind("(")] if name.endswith(")") else name)[-90:]
            lines.append(f"timed | {short} | {len(t)} | {sum(t) / len(t):.0f} | {t[len(t) // 2]}")
    out = os.path.join(PROFILES, f"kernels_{workload}_kernel_stats.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


KERNEL_KEYS = ("chunk_scan_fused", "one_chunk", "chunk_output", "chunk_state", "state_pass", "chunk_cumsum",
               "empty_sequence", "state_correction")
# fp32 inputs run v_mfma_f32_16x16x4_f32 (2048 flops), bf16 v_mfma_f32_16x16x32_bf16 (16384).
MFMA_FLOPS = {"bf16": 16384, "f32": 2048}
N_SIMDS, N_SE = 1024, 32


def _kernel_key(symbol):
    """The step a kernel symbol belongs to (the state at index runs the generic
    chunk_state kernel and is counted with it)."""
    for key in KERNEL_KEYS:
        if re.search(rf"(?<![a-z_]){key}(_heads|_dma)?_kernel", symbol):
            return key
    return None


def summarize_pmc(dirs, workload=HEADLINE, commands=()):
    """Per kernel of one workload: the median per dispatch of every counter
    found under `dirs` (rows of one dispatch summed), FETCH_SIZE / WRITE_SIZE
    turned into bytes with the copy probe's factor, and the derived figures."""
    per = {}   # kernel key -> counter -> dispatch -> value
    symbols = {}
    for d in dirs:
        _, rows = _read_csv(os.path.join(d, "**", "*counter_collection.csv"))
        for r in rows:
            sym = r.get("Kernel_Name", "")
            key = "copy" if "copy" in sym.lower() else _kernel_key(sym)
            if key is None:
                continue
            symbols.setdefault(key, sym)
            disp = (d, int(r.get("Dispatch_Id") or 0))
            c = per.setdefault(key, {}).setdefault(r["Counter_Name"], {})
            c[disp] = c.get(disp, 0.0) + float(r["Counter_Value"])

    def med(key, counter):
        vals = sorted(per.get(key, {}).get(counter, {}).values())
        return vals[len(vals) // 2] if vals else None

    wl = ALL_WORKLOADS[workload]
    copy_bytes = 256 << 20
    # The copy probe runs last: its three 256 MiB copies are the last three
    # copy dispatches of each run (earlier ones upload the inputs).
    def copy_factor(counter):
        disp = per.get("copy", {}).get(counter, {})
        last = {}
        for (d, i), v in disp.items():
            last.setdefault(d, []).append((i, v))
        vals = sorted(v for runs in last.values() for _, v in sorted(runs)[-3:])
        return copy_bytes / (vals[len(vals) // 2] * 1024.0) if vals else None

    fc, wc = copy_factor("FETCH_SIZE"), copy_factor("WRITE_SIZE")
    kb = kernel_bytes(wl)
    for key in per:
        if key == "copy":
            continue
        c = {k: med(key, k) for k in per[key]}
        sym = symbols[key]
        lines = [f"# rocprofv3 --pmc counters of {key} on {workload} (medians per dispatch; a dispatch's rows summed)",
                 f"# kernel symbol: {sym[:sym.rfind('(')] if sym.endswith(')') else sym}"]
        lines += [f"# command: {cmd}" for cmd in commands]
        lines += [f"kernel_source_sha256 = {source_hash(key)}"]
        for k in sorted(c):
            lines.append(f"{k} = {c[k]:.0f}")
        ab = kb.get(key)
        if c.get("FETCH_SIZE") is not None and c.get("WRITE_SIZE") is not None and fc and wc:
            fb, wb = c["FETCH_SIZE"] * 1024.0 * fc, c["WRITE_SIZE"] * 1024.0 * wc
            lines += ["# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by 256 MiB over what",
                      "# the same counter reads for a plain 256 MiB device copy in the same run",
                      f"copy_factor_fetch = {fc:.4f}", f"copy_factor_write = {wc:.4f}",
                      f"fetch_bytes_per_launch = {fb:.0f}", f"write_bytes_per_launch = {wb:.0f}",
                      f"traffic_bytes_per_launch = {fb + wb:.0f}"]
            if ab:
                lines += [f"algorithmic_bytes_per_launch = {ab}", f"traffic_over_algorithmic = {(fb + wb) / ab:.3f}"]
        t_us = timed_mean_us(key, workload)
        if t_us and ab:
            gbs = ab / (t_us * 1e-6) / 1e9
            lines += [f"# against MI355X peaks, with the kernel's mean duration in kernels_{workload}_kernel_stats.txt",
                      f"mean_duration_us = {t_us:.2f}",
                      f"algorithmic_GBps = {gbs:.1f}", f"algorithmic_frac_of_hbm_peak = {gbs / PEAK_HBM_GBS:.4f}"]
            if c.get("FETCH_SIZE") is not None and c.get("WRITE_SIZE") is not None and fc and wc:
                tb = c["FETCH_SIZE"] * 1024.0 * fc + c["WRITE_SIZE"] * 1024.0 * wc
                lines.append(f"traffic_GBps = {tb / (t_us * 1e-6) / 1e9:.1f}")
            kf = kernel_flops(wl).get(key)
            if kf:
                peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
                tf = kf / (t_us * 1e-6) / 1e12
                lines += [f"algorithmic_flops_per_launch_kernel = {kf}", f"algorithmic_TFLOPs = {tf:.1f}",
                          f"algorithmic_frac_of_mfma_peak = {tf / peak:.4f}"]
        if c.get("SQ_INSTS_MFMA") == 0:
            lines.append("# no MFMA instructions: this kernel computes on the vector ALUs")
        elif c.get("SQ_INSTS_MFMA") is not None:
            ex = c["SQ_INSTS_MFMA"] * MFMA_FLOPS[wl.dtype]
            lines += [f"# executed MFMA flops = SQ_INSTS_MFMA x {MFMA_FLOPS[wl.dtype]} flops per instruction",
                      f"mfma_flops_executed = {ex:.0f}"]
            if key in ("chunk_scan_fused", "one_chunk"):
                alg = total_flops(wl)
                lines += [f"algorithmic_flops_per_launch = {alg}", f"executed_over_algorithmic = {ex / alg:.3f}"]
        if c.get("SQ_VALU_MFMA_BUSY_CYCLES") is not None and c.get("SQ_BUSY_CYCLES"):
            # SQ_BUSY_CYCLES sums the 32 shader engines; the MFMA busy counter sums the 1024 SIMDs.
            se_cycles = c["SQ_BUSY_CYCLES"] / N_SE
            lines += ["# MFMA busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x SQ_BUSY_CYCLES / 32 SEs)",
                      f"mfma_busy_frac = {c['SQ_VALU_MFMA_BUSY_CYCLES'] / (N_SIMDS * se_cycles):.4f}"]
        if c.get("SQ_WAIT_ANY") is not None and c.get("SQ_WAVE_CYCLES"):
            lines.append(f"wait_any_over_wave_cycles = {c['SQ_WAIT_ANY'] / c['SQ_WAVE_CYCLES']:.4f}")
        if c.get("SQ_LDS_BANK_CONFLICT") is not None and c.get("SQ_ACTIVE_INST_LDS"):
            lines.append(f"lds_bank_conflict_over_active_lds = "
                         f"{c['SQ_LDS_BANK_CONFLICT'] / c['SQ_ACTIVE_INST_LDS']:.4f}")
        out = os.path.join(PROFILES, f"{key}_{workload}_counters.txt")
        with open(out, "w") as f:
            f.write("\n".join(lines) + "\n")
        print(out)


# --------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # ~0.2 s of untimed steps: the GPU's clocks ramp up over the first milliseconds.
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--cold-steps", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(ALL_WORKLOADS))
    ap.add_argument("--state-correction-only", action="store_true",
                    help="time ssd_state_correction on a sequence shard and print its figures")
    ap.add_argument("--path", default="auto", choices=["auto", "one_chunk", "single_pass", "chunk_parallel"])
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads and the decode line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR")
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--command", action="append", default=[], help="command line recorded in a profile summary")
    args = ap.parse_args()

    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc, workload=args.workload, commands=args.command)
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats, workload=args.workload, command=" ".join(args.command),
                               steps=args.steps, warmup=args.warmup, cold_steps=args.cold_steps)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the SSD forward here runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built). Run with --gpus 1.", file=sys.stderr)
        raise SystemExit(2)

    import torch

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)

    if args.state_correction_only:
        print(json.dumps(time_state_correction(args.steps, args.warmup, device)), flush=True)
        if args.copy_probe:
            copy_probe(device)
        return
    wl = ssd_inputs.WORKLOADS[args.workload]
    inp, res = time_workload(wl, args.steps, args.warmup, device, args.path, args.cold_steps)
    ms = res["ms_per_step"]
    flops = total_flops(wl)
    tflops = flops / (ms * 1e-3) / 1e12

    workloads = {}
    if not args.headline_only:
        for name in ssd_inputs.WORKLOAD_ORDER:
            if name == wl.name:
                continue
            w2 = ssd_inputs.WORKLOADS[name]
            _, r2 = time_workload(w2, max(10, args.steps // 4), max(10, args.warmup // 4), device, "auto", 5)
            m2 = r2["ms_per_step"]
            workloads[name] = {"path": r2["path"], "kernels": r2["kernels"], "ms_per_step": round(m2, 5),
                               "tokens_per_s": round(w2.tokens / (m2 * 1e-3), 1),
                               "TFLOP/s": round(total_flops(w2) / (m2 * 1e-3) / 1e12, 2),
                               "step_bytes": step_bytes(w2),
                               "hbm_frac": round(step_bytes(w2) / (m2 * 1e-3) / (PEAK_HBM_GBS * 1e9), 4),
                               "warm": r2["warm"], "cold": r2["cold"]}

    decode = None if args.headline_only else time_decode(max(20, args.steps // 2), 5, device)
    correction = None if args.headline_only else time_state_correction(max(20, args.steps // 2), 20, device)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl, inp)
    line = {
        "metric": METRIC,
        "value": round(wl.tokens / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded counter-based generator; inputs resident in HBM)",
        "config": {"workload": wl.name, "batch": wl.batch, "seqlen": wl.seqlen, "nheads": wl.nheads,
                   "headdim": wl.headdim, "dstate": wl.dstate, "ngroups": wl.ngroups, "chunk": wl.chunk,
                   "path": res["path"], "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "alg_flops_per_step": flops,
        "timing": {"source": "HIP events on the library's stream: warm, one before the first step and one after "
                             "each of up to 10 groups of back-to-back steps (mean over all steps; median and min "
                             "over the groups' means); cold, one pair around each step after a 512 MiB flush",
                   "warm": res["warm"], "cold": dict(res["cold"], flush_bytes=FLUSH_BYTES),
                   "wall_s": round(res["wall_s"], 4)},
        "roofline": roofline_entry(wl, res),
        "cpu_baseline": cpu,
        "kernels": res["kernels"],
        "workloads": workloads,
        "decode": decode,
        "state_correction": correction,
        "input_sha256": inp.sha256,
    }
    if args.copy_probe:
        copy_probe(device)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
