"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP path through the C ABI, run the oracle, and measure errors."""
from __future__ import annotations

import numpy as np
import torch

import mamba_ssd_scan_06_amd as ssd
import oracle
import ssd_inputs

# Max relative error bounds (normwise: max |gpu - oracle| / max |oracle|) per
# output tensor, as fixed for bf16 and fp32 inputs; states are fp32 in both.
TOL = {"bf16": 2e-2, "f32": 1e-4}


def workload(name, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype="bf16", init_state=False,
             state_out=False, seed=7):
    return ssd_inputs.Workload(name, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, dtype,
                               init_state=init_state, state_out=state_out, seed=seed)


def relerr(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), "non-finite values in GPU output"
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (scale if scale > 0 else 1.0)


def _bf16(bits, device):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def device_inputs(inp: ssd_inputs.Inputs, device="cuda"):
    if inp.wl.dtype == "bf16":
        x, B, C = (_bf16(getattr(inp, k + "_bits"), device) for k in ("x", "B", "C"))
    else:
        x, B, C = (torch.from_numpy(np.ascontiguousarray(getattr(inp, k))).to(device) for k in ("x", "B", "C"))
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(x=x, dt=t(inp.dt), A=t(inp.A), B=B, C=C, D=t(inp.D), init_state=t(inp.init_state),
                state_out_idx=t(inp.state_out_idx))


def to_np(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy().astype(np.float64)


def gpu_run(inp, chunk=None, use_D=True, use_init=True, use_state_out=True, dev=None, return_workspace=False,
            path=ssd.SSD_PATH_AUTO, outputs=None):
    """One call through the C ABI.  With return_workspace the call runs the
    chunk-parallel path (the only one with a workspace) on a zero-filled
    workspace and the intermediates it writes are returned too.  `outputs`
    may hold caller-allocated y / final_state / state_out tensors."""
    dev = dev or device_inputs(inp)
    chunk = chunk or inp.wl.chunk
    b, T, H, P = dev["x"].shape
    G, N = dev["B"].shape[2], dev["B"].shape[3]
    code = ssd.SSD_DTYPE_BF16 if inp.wl.dtype == "bf16" else ssd.SSD_DTYPE_F32
    shape = ssd.make_shape(b, T, H, P, N, G)
    ws = None
    if return_workspace:
        path = ssd.SSD_PATH_CHUNK_PARALLEL
        lay = ssd.ssd_get_workspace_layout(shape, chunk, code)
        ws = torch.zeros(max(lay.total_bytes, 1), dtype=torch.uint8, device=dev["x"].device)
    outputs = outputs or {}
    y, fin, sout, names = ssd.ssd_chunk_scan_fwd_ex(
        dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"] if use_D else None,
        dev["init_state"] if use_init else None, chunk,
        dev["state_out_idx"] if use_state_out else None, path=path, workspace=ws, **outputs)
    torch.cuda.synchronize()
    out = dict(y=to_np(y), final=to_np(fin), state_out=to_np(sout))
    if return_workspace:
        v = ssd.workspace_views(ws, shape, chunk, code)
        for k in ("cs", "ct", "dte", "states"):
            out[k] = to_np(v[k])
        # prev entry 0 is written only with an initial state.
        first = 0 if (use_init and dev["init_state"] is not None) else 1
        out["prev"] = to_np(v["prev"][:, first:])
    return out


def kernel_names(inp, chunk=None, dev=None, path=ssd.SSD_PATH_AUTO):
    """Names of the kernels one call launches (through the timing marks of
    ssd_chunk_scan_fwd_ex)."""
    dev = dev or device_inputs(inp)
    chunk = chunk or inp.wl.chunk
    evs = [torch.cuda.Event() for _ in range(8)]
    for e in evs:
        e.record()  # creates the event
    torch.cuda.synchronize()
    *_, names = ssd.ssd_chunk_scan_fwd_ex(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"],
                                          dev["init_state"], chunk, dev["state_out_idx"], path=path,
                                          marks=[e.cuda_event for e in evs])
    torch.cuda.synchronize()
    return names


def oracle_run(inp, use_D=True, use_init=True, use_state_out=True, chunk=0):
    y, fin, sout, cst = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D if use_D else None,
                                           inp.init_state if use_init else None,
                                           inp.state_out_idx if use_state_out else None, chunk=chunk)
    return dict(y=y, final=fin, state_out=sout, chunk_states=cst)
