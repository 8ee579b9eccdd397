#!/usr/bin/env python
"""Throughput of the SSD chunked-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one full forward (chunk cumsum, chunk states, state passing,
chunk outputs with the state-to-output term and D skip, and the state at the
accepted index where the workload asks for it) over one batch of seeded
synthetic inputs already resident in HBM.  The headline workload is the
Mamba-2 2.7B layer shape (b=8, T=2048, H=80, P=64, N=128, G=1, Q=256, bf16
in, fp32 state); the other four workloads are timed too and reported under
"workloads".  Prints ONE JSON line.

Per-kernel durations are measured live with HIP events that the library
records between its kernels (ssd_chunk_scan_fwd_marked) on the stream the
kernels run on, over the timed steps.  The roofline entry is for the kernel
with the largest average duration; its algorithmic bytes and flops per
launch are computed below from the problem sizes.  HBM traffic comes from
the rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/ when it was
taken on the current kernel source (else null).

Other modes:
    --copy-probe            also run a plain 256 MiB device copy (counter calibration)
    --summarize-pmc F W     turn two rocprofv3 --pmc output dirs into a profiles/ summary
    --summarize-stats D     turn a rocprofv3 --kernel-trace --stats dir into a profiles/ summary
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
    "state_at_index": ["chunk_state.hip", "device_common.hpp"],
}
CSRC = os.path.join(ROOT, "mamba_ssd_scan_06_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# ------------------------------------------------------------ work per kernel
def chunk_lengths(wl):
    Q, T = wl.chunk, wl.seqlen
    return [min(Q, T - c) for c in range(0, T, Q)]


def algorithmic_work(wl, idx=None):
    """Minimal HBM bytes and algorithmic flops of each kernel for one call.

    Bytes count each tensor a kernel must read or write once: inputs in their
    dtype, the per-token tables (cs, ct, dte) and chunk states in fp32, the
    states entering each chunk in the input dtype.  Flops count the causal
    triangle only and C.B^T once per (b, chunk, group), not per head."""
    b, T, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    e = 2 if wl.dtype == "bf16" else 4
    nc = len(chunk_lengths(wl))
    x = b * T * H * P * e
    bc = b * T * G * N * e
    dt = b * T * H * 4
    tab = b * H * nc * wl.chunk * 4      # one per-token table
    st = b * H * P * N * 4               # one fp32 state per (b, h)
    S = nc * st                          # chunk states, fp32
    prev_chunks = nc if wl.init_state else nc - 1
    prev = prev_chunks * st // 4 * e     # states entering chunks, input dtype
    qs = chunk_lengths(wl)
    work = {
        "chunk_cumsum": dict(bytes=dt + 3 * tab, flops=b * T * H),
        "chunk_state": dict(bytes=x + bc + dt + tab + S, flops=2 * b * H * sum(qs) * N * P),
        "state_pass": dict(bytes=S + prev + st + (st if wl.init_state else 0), flops=2 * b * nc * H * P * N),
        "chunk_output": dict(
            bytes=2 * x + 2 * bc + 3 * tab + prev,
            flops=b * sum(G * q * (q + 1) * N + H * q * (q + 1) * P for q in qs)
            + 2 * b * H * N * P * sum(q for c, q in enumerate(qs) if c > 0 or wl.init_state)),
    }
    # single pass: x, B, C and the tables read once, y and the states written once
    work["chunk_scan_fused"] = dict(
        bytes=2 * x + 2 * bc + 3 * tab + (st if wl.init_state else 0) + st + (st if wl.state_out else 0),
        flops=work["chunk_state"]["flops"] + work["chunk_output"]["flops"])
    if 1 <= T <= 32 and nc == 1:
        # one fused kernel: h0 read once, both states written once
        toks = [min(j, T - 1) + 1 if j >= 0 else 0 for j in (idx if idx is not None else [])] if wl.state_out else []
        work["one_chunk"] = dict(
            bytes=2 * x + 2 * bc + dt + (st if wl.init_state else 0) + st + (st if wl.state_out else 0),
            flops=b * (G * T * (T + 1) * N + H * T * (T + 1) * P) + 4 * b * H * P * N * T
            + 2 * H * P * N * sum(toks))
    if wl.state_out:
        Q = wl.chunk
        toks = [(j % Q) + 1 if j >= 0 else 0 for j in (idx if idx is not None else [])]
        work["state_at_index"] = dict(
            bytes=sum(t * (H * P * e + G * N * e + H * 4) for t in toks) + b * H * Q * 4 + 2 * st,
            flops=2 * H * N * P * sum(toks))
    return work


def total_flops(wl):
    qs = chunk_lengths(wl)
    b, H, P, N, G = wl.batch, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    return b * sum(G * q * (q + 1) * N + H * q * (q + 1) * P + 4 * H * q * N * P for q in qs)


def source_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES.get(kernel, []):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------- HIP events
class HipEvents:
    """hipEventCreate / hipEventElapsedTime through the HIP runtime torch loaded."""

    def __init__(self):
        import torch  # noqa: F401  (torch's runtime is the one libssd binds to)
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(ev.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


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


def time_workload(wl, steps, warmup, device, events):
    """Returns (inputs, result dict) for `steps` timed forwards of `wl`."""
    import torch

    import mamba_ssd_scan_06_amd as ssd

    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp, device)
    b, T, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    code = ssd.SSD_DTYPE_BF16 if wl.dtype == "bf16" else ssd.SSD_DTYPE_F32
    shape = ssd.make_shape(b, T, H, P, N, G)
    ws = torch.empty(ssd.ssd_workspace_bytes(shape, wl.chunk, code), dtype=torch.uint8, device=device)
    y = torch.empty_like(dev["x"])
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device=device)
    sout = torch.empty_like(fin) if wl.state_out else None
    args = (dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["init_state"], wl.chunk,
            dev["state_out_idx"])
    kw = dict(y=y, final_state=fin, state_out=sout, workspace=ws)
    for _ in range(warmup):
        ssd.ssd_chunk_scan_fwd(*args, **kw)
    # Whole steps, back to back, with events only around the timed region.
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        ssd.ssd_chunk_scan_fwd(*args, **kw)
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / steps
    # Per-kernel durations: the same steps again, with HIP events recorded on
    # the kernels' stream between kernels.
    nk = 5 if wl.state_out else 4
    marks = [events.create(nk + 1) for _ in range(steps)]
    names = None
    for k in range(steps):
        _, _, _, names = ssd.ssd_chunk_scan_fwd_marked(*args, marks=marks[k], **kw)
    torch.cuda.synchronize()
    per_kernel = {}
    for i, name in enumerate(names):
        per_kernel[name] = sum(events.elapsed_ms(m[i], m[i + 1]) for m in marks) / steps
    for m in marks:
        events.destroy(m)
    return inp, dict(ms_per_step=ms_step, wall_s=wall, kernel_ms=per_kernel, kernel_order=names)


def roofline_entry(wl, name, ms, work, traffic):
    w = work[name]
    ai = w["flops"] / w["bytes"]
    peak_flops = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    ridge = peak_flops * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge:
        achieved = w["flops"] / (ms * 1e-3) / 1e12
        return {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2), "peak": peak_flops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_flops, 4), "traffic": traffic,
                "alg_bytes": w["bytes"], "alg_flops": w["flops"], "avg_ms": round(ms, 5)}
    achieved = w["bytes"] / (ms * 1e-3) / 1e9
    return {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic, "alg_bytes": w["bytes"],
            "alg_flops": w["flops"], "avg_ms": round(ms, 5)}


def traffic_from_profile(kernel, workload):
    """HBM bytes per launch from profiles/<kernel>_<workload>_hbm_traffic.txt, if
    the counters were taken on the current kernel source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != source_hash(kernel):
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


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


def cpu_baseline(wl, inp):
    import oracle

    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state, inp.state_out_idx,
                       nthreads=cores)
    dt = time.perf_counter() - t0
    return {"value": round(wl.tokens / dt, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the full {wl.name} workload ({wl.tokens} tokens), fp64 recurrence, one pass, "
                      f"{dt:.2f} s wall on {cores} threads"}


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


def summarize_stats(d, workload=HEADLINE, command=""):
    files, rows = _read_csv(os.path.join(d, "**", "*kernel_stats.csv"))
    if not rows:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    lines = [f"# rocprofv3 kernel-trace statistics, workload {workload}", f"# command: {command}",
             f"# source: {', '.join(os.path.relpath(f, ROOT) for f in files)}",
             "# name | calls | total_ns | avg_ns | min_ns | max_ns | pct"]
    for r in sorted(rows, key=lambda r: -float(r.get("TotalDurationNs", 0))):
        name = r.get("Name", "")
        short = (name[:name.rfind("(")] if name.endswith(")") else name)[-90:]
        lines.append(f"{short} | {r.get('Calls')} | {r.get('TotalDurationNs')} | {float(r.get('AverageNs', 0)):.0f} | "
                     f"{r.get('MinNs')} | {r.get('MaxNs')} | {float(r.get('Percentage', 0)):.2f}")
    out = os.path.join(PROFILES, f"kernels_{workload}_kernel_stats.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out)


def summarize_pmc(fetch_dir, write_dir, workload=HEADLINE, command=""):
    def per_kernel(d, counter):
        _, rows = _read_csv(os.path.join(d, "**", "*counter_collection.csv"))
        vals = {}
        for r in rows:
            if r.get("Counter_Name") != counter:
                continue
            vals.setdefault(r.get("Kernel_Name", ""), []).append(float(r.get("Counter_Value", 0)))
        return vals

    fetch = per_kernel(fetch_dir, "FETCH_SIZE")
    write = per_kernel(write_dir, "WRITE_SIZE")
    copy_bytes = 256 << 20

    def find(d, key):
        # kernel symbols look like "...chunk_output_heads_kernel<8, 4, 16, true>(...)"; the
        # step's kernel is the matching one with the most dispatches
        pat = re.compile(rf"(?<![a-z_]){re.escape(key)}(_heads|_dma)?_kernel") if key != "copy" else None
        hits = {k: v for k, v in d.items() if (pat.search(k) if pat else key in k)}
        return max(hits.items(), key=lambda kv: len(kv[1])) if hits else (None, None)

    _, cf = find(fetch, "copy")
    _, cw = find(write, "copy")
    if not cf or not cw:
        raise SystemExit("copy probe kernel not found in counter output")
    f_copy = copy_bytes / (sorted(cf)[len(cf) // 2] * 1024.0)
    w_copy = copy_bytes / (sorted(cw)[len(cw) // 2] * 1024.0)
    wl = ssd_inputs.WORKLOADS[workload]
    work = algorithmic_work(wl)
    for kernel in ("chunk_scan_fused", "chunk_output", "chunk_state", "state_pass", "chunk_cumsum"):
        kf_name, kf = find(fetch, kernel)
        _, kw = find(write, kernel)
        if not kf or not kw:
            continue
        fb = sorted(kf)[len(kf) // 2] * 1024.0 * f_copy
        wb = sorted(kw)[len(kw) // 2] * 1024.0 * w_copy
        out = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_traffic.txt")
        with open(out, "w") as f:
            f.write(f"# HBM traffic of {kernel} on {workload} from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE\n")
            f.write(f"# command: {command}\n")
            f.write(f"# kernel symbol: {kf_name[:kf_name.rfind('(')] if kf_name.endswith(')') else kf_name}\n")
            f.write("# counters are KiB per dispatch; each is scaled by (256 MiB / what the same counter reads\n")
            f.write("# for a plain 256 MiB device copy in the same run); medians over dispatches\n")
            f.write(f"kernel_source_sha256 = {source_hash(kernel)}\n")
            f.write(f"copy_factor_fetch = {f_copy:.4f}\n")
            f.write(f"copy_factor_write = {w_copy:.4f}\n")
            f.write(f"fetch_bytes_per_launch = {fb:.0f}\n")
            f.write(f"write_bytes_per_launch = {wb:.0f}\n")
            f.write(f"traffic_bytes_per_launch = {fb + wb:.0f}\n")
            f.write(f"algorithmic_bytes_per_launch = {work[kernel]['bytes']}\n")
            f.write(f"traffic_over_algorithmic = {(fb + wb) / work[kernel]['bytes']:.3f}\n")
        print(out)


# --------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=HEADLINE, choices=list(ssd_inputs.WORKLOADS))
    ap.add_argument("--headline-only", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-stats", metavar="DIR")
    ap.add_argument("--command", default="", help="command line recorded in a profile summary")
    args = ap.parse_args()

    if args.summarize_pmc:
        return summarize_pmc(*args.summarize_pmc, workload=args.workload, command=args.command)
    if args.summarize_stats:
        return summarize_stats(args.summarize_stats, workload=args.workload, command=args.command)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the SSD forward here runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built). Run with --gpus 1.", file=sys.stderr)
        raise SystemExit(2)

    import torch

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    events = HipEvents()

    wl = ssd_inputs.WORKLOADS[args.workload]
    inp, res = time_workload(wl, args.steps, args.warmup, device, events)
    work = algorithmic_work(wl, inp.state_out_idx)
    ms = res["ms_per_step"]
    flops = total_flops(wl)
    tflops = flops / (ms * 1e-3) / 1e12
    dominant = max(res["kernel_ms"], key=res["kernel_ms"].get)
    roof = roofline_entry(wl, dominant, res["kernel_ms"][dominant], work,
                          traffic_from_profile(dominant, wl.name))
    kernels = {}
    for name, kms in res["kernel_ms"].items():
        w = work.get(name, {"bytes": 0, "flops": 0})
        kernels[name] = {"avg_us": round(kms * 1e3, 2), "alg_bytes": w["bytes"], "alg_flops": w["flops"],
                         "GB/s": round(w["bytes"] / (kms * 1e-3) / 1e9, 1),
                         "TFLOP/s": round(w["flops"] / (kms * 1e-3) / 1e12, 2)}

    workloads = {}
    if not args.headline_only:
        for name in ssd_inputs.WORKLOAD_ORDER:
            if name == wl.name:
                continue
            w2 = ssd_inputs.WORKLOADS[name]
            inp2, r2 = time_workload(w2, max(10, args.steps // 4), max(3, args.warmup // 2), device, events)
            m2 = r2["ms_per_step"]
            work2 = algorithmic_work(w2, inp2.state_out_idx)
            workloads[name] = {"ms_per_step": round(m2, 5), "tokens_per_s": round(w2.tokens / (m2 * 1e-3), 1),
                               "TFLOP/s": round(total_flops(w2) / (m2 * 1e-3) / 1e12, 2),
                               "alg_GB/s": round(sum(work2[k]["bytes"] for k in r2["kernel_ms"]) / (m2 * 1e-3) / 1e9,
                                                 1),
                               "kernel_us": {k: round(v * 1e3, 2) for k, v in r2["kernel_ms"].items()}}
            del inp2

    decode = None if args.headline_only else time_decode(max(20, args.steps // 2), 5, device)
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
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "alg_flops_per_step": flops,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "workloads": workloads,
        "decode": decode,
        "input_sha256": inp.sha256,
    }
    if args.copy_probe:
        copy_probe(device)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
