"""Sequence sharding through ssd_state_correction, against the oracle's run
over the whole sequence.

A sequence is cut into shards.  The first runs from the sequence's initial
state; every later one runs from a zero state and is then corrected with the
state entering it (the previous shard's final state), which is the one-GPU
step of context parallelism ("Transformers are SSMs" article,
cloud.tencent.com.cn, section "序列并行的两种形式").  The corrected outputs,
final state and state after the accepted index must match the oracle's
single run within the dtype's tolerance."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_06_amd as ssd
import oracle
import ssd_inputs
from ssd_testing import TOL, device_inputs, relerr, to_np, workload

pytestmark = pytest.mark.gpu


def _slice(dev, lo, hi):
    """Token range [lo, hi) of the token-major device inputs."""
    out = dict(dev)
    for k in ("x", "dt", "B", "C"):
        out[k] = dev[k][:, lo:hi].contiguous()
    return out


def run_sharded(inp, cuts, j_full, chunk):
    """Forward over shards [cuts[k], cuts[k+1]) with the state carried by
    ssd_state_correction; returns y, the final state and the state after
    each sequence's accepted index j_full[b] (numpy, fp64)."""
    dev = device_inputs(inp)
    b = dev["x"].shape[0]
    ys, h_in, sout = [], dev["init_state"], None
    jt = torch.as_tensor(j_full, dtype=torch.int32)
    for k in range(len(cuts) - 1):
        lo, hi = cuts[k], cuts[k + 1]
        sh = _slice(dev, lo, hi)
        # The accepted index relative to the shard: -1 is the state entering
        # it; indices before that belong to an earlier shard.
        jl = (jt - lo).clamp(min=-1)
        in_shard = (jt >= lo - 1) & (jt < hi) if k < len(cuts) - 2 else (jt >= lo - 1)
        jl_dev = jl.to(dev["x"].device)
        first = k == 0
        y, fin, so = ssd.ssd_chunk_scan_fwd(sh["x"], sh["dt"], sh["A"], sh["B"], sh["C"], sh["D"],
                                            h_in if first else None, chunk, jl_dev)
        if not first:
            ssd.ssd_state_correction(y, sh["dt"], sh["A"], sh["C"], h_in, shard_final=fin, final_state=fin,
                                     state_out_idx=jl_dev, state_out=so)
        ys.append(y)
        mask = in_shard.to(so.device).view(b, 1, 1, 1)
        sout = so.clone() if sout is None else torch.where(mask, so, sout)
        h_in = fin
    torch.cuda.synchronize()
    return to_np(torch.cat(ys, dim=1)), to_np(h_in), to_np(sout)


CASES = [
    # name, b, T, H, P, N, G, chunk, dtype, cuts
    ("bf16_two_shards", 2, 300, 4, 64, 128, 2, 64, "bf16", [0, 130, 300]),
    ("bf16_dstate256_headdim128", 1, 200, 2, 128, 256, 1, 64, "bf16", [0, 77, 200]),
    ("f32_dstate16_headdim16", 1, 150, 3, 16, 16, 1, 32, "f32", [0, 50, 150]),
    ("bf16_groups_three_shards", 3, 229, 8, 32, 64, 4, 32, "bf16", [0, 64, 65, 229]),
    ("f32_headdim128_four_shards", 2, 257, 2, 128, 32, 2, 64, "f32", [0, 1, 100, 192, 257]),
    ("bf16_empty_shard", 1, 96, 2, 64, 128, 1, 32, "bf16", [0, 40, 40, 96]),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_sharded_forward_matches_oracle(case):
    name, b, T, H, P, N, G, chunk, dtype, cuts = case
    wl = workload(name, b, T, H, P, N, G, chunk, dtype, init_state=True, state_out=True, seed=31)
    inp = ssd_inputs.generate(wl)
    # One accepted index per sequence, in the last shard or at its entry.
    rng = np.random.default_rng(5)
    j_full = rng.integers(cuts[-2] - 1, T, size=b).astype(np.int32)
    y_ref, fin_ref, sout_ref, _ = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state,
                                                     j_full)
    y, fin, sout = run_sharded(inp, cuts, j_full, chunk)
    tol = TOL[dtype]
    assert relerr(y, y_ref) <= tol, relerr(y, y_ref)
    assert relerr(fin, fin_ref) <= tol, relerr(fin, fin_ref)
    assert relerr(sout, sout_ref) <= tol, relerr(sout, sout_ref)


def test_shard_of_long_sequence_workload():
    """A 2048-token shard of the 16K-token dstate-256 workload (its share on
    8 GPUs), after a shard of the same length."""
    wl = workload("long_shard", 1, 4096, 64, 64, 256, 1, 256, "bf16", init_state=True, state_out=True, seed=41)
    inp = ssd_inputs.generate(wl)
    j_full = np.array([3000], dtype=np.int32)
    y_ref, fin_ref, sout_ref, _ = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state,
                                                     j_full)
    y, fin, sout = run_sharded(inp, [0, 2048, 4096], j_full, 256)
    assert relerr(y[:, 2048:], y_ref[:, 2048:]) <= TOL["bf16"]
    assert relerr(fin, fin_ref) <= TOL["bf16"]
    assert relerr(sout, sout_ref) <= TOL["bf16"]
    # (After 2048 tokens of these decays the entering state adds under 1% to
    # the outputs and the final state, so this case checks the plumbing at the
    # real shard shape; the correction term itself is checked against the
    # pure decay in test_correction_term_is_the_pure_decay.)


TERM_CASES = [
    # name, b, T, H, P, N, G, dtype  (few items: many token ranges per item)
    ("bf16_ranges", 1, 1000, 2, 64, 128, 1, "bf16"),
    ("f32_ranges_dstate16", 2, 333, 2, 16, 16, 2, "f32"),
    ("bf16_dstate256_headdim128", 2, 700, 4, 128, 256, 2, "bf16"),
    ("f32_headdim32_dstate64", 1, 64, 3, 32, 64, 1, "f32"),
    ("bf16_one_token", 3, 1, 4, 64, 128, 4, "bf16"),
]


@pytest.mark.parametrize("case", TERM_CASES, ids=[c[0] for c in TERM_CASES])
def test_correction_term_is_the_pure_decay(case):
    """With y and the shard's final state zero, the call leaves exactly the
    contribution of h_in: the outputs and states of the recurrence from h_in
    with x = 0 (pure decay), as the oracle computes them."""
    name, b, T, H, P, N, G, dtype = case
    wl = workload(name, b, T, H, P, N, G, 64, dtype, init_state=True, state_out=True, seed=77)
    inp = ssd_inputs.generate(wl)
    inp.init_state = inp.init_state * 10.0  # a state of unit scale
    zero_x = np.zeros_like(inp.x)
    y_ref, fin_ref, sout_ref, _ = oracle.ssd_forward(zero_x, inp.dt, inp.A, inp.B, inp.C, None, inp.init_state,
                                                     inp.state_out_idx)
    dev = device_inputs(inp)
    y = torch.zeros_like(dev["x"])
    zero = torch.zeros_like(dev["init_state"])
    fin = torch.empty_like(zero)
    so = torch.zeros_like(zero)
    ssd.ssd_state_correction(y, dev["dt"], dev["A"], dev["C"], dev["init_state"], shard_final=zero,
                             final_state=fin, state_out_idx=dev["state_out_idx"], state_out=so)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert relerr(to_np(y), y_ref) <= tol, relerr(to_np(y), y_ref)
    assert relerr(to_np(fin), fin_ref) <= tol, relerr(to_np(fin), fin_ref)
    assert relerr(to_np(so), sout_ref) <= tol, relerr(to_np(so), sout_ref)


def test_zero_token_shard_and_in_place_final():
    """T = 0: final = shard_final + h_in (in place), state_out += h_in."""
    dev = torch.device("cuda")
    b, H, P, N, G = 2, 4, 64, 128, 1
    g = torch.Generator().manual_seed(3)
    h_in = torch.randn(b, H, P, N, generator=g).to(dev)
    fin0 = torch.randn(b, H, P, N, generator=g).to(dev)
    so0 = torch.randn(b, H, P, N, generator=g).to(dev)
    expect_fin = (fin0 + h_in).cpu()
    expect_so = (so0 + h_in).cpu()
    y = torch.empty(b, 0, H, P, dtype=torch.bfloat16, device=dev)
    C = torch.empty(b, 0, G, N, dtype=torch.bfloat16, device=dev)
    dt = torch.empty(b, 0, H, dtype=torch.float32, device=dev)
    A = -torch.ones(H, dtype=torch.float32, device=dev)
    idx = torch.tensor([0, -1], dtype=torch.int32, device=dev)
    ssd.ssd_state_correction(y, dt, A, C, h_in, shard_final=fin0, final_state=fin0, state_out_idx=idx,
                             state_out=so0)
    torch.cuda.synchronize()
    assert torch.equal(fin0.cpu(), expect_fin)
    assert torch.equal(so0.cpu(), expect_so)


def test_correction_is_deterministic_and_writes_only_its_outputs():
    """Three identical calls give identical bits; NaN canaries around y and
    the states stay untouched."""
    wl = workload("det", 2, 200, 4, 64, 128, 1, 64, "bf16", init_state=True, state_out=True, seed=9)
    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp)
    b, T, H, P = dev["x"].shape
    N = dev["B"].shape[3]
    y0, fin0, so0 = ssd.ssd_chunk_scan_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], None,
                                           64, dev["state_out_idx"])
    outs = []
    for _ in range(3):
        pad = 64
        ybuf = torch.full((y0.numel() + 2 * pad,), float("nan"), dtype=y0.dtype, device=y0.device)
        fbuf = torch.full((fin0.numel() + 2 * pad,), float("nan"), dtype=torch.float32, device=y0.device)
        sbuf = torch.full((so0.numel() + 2 * pad,), float("nan"), dtype=torch.float32, device=y0.device)
        y = ybuf[pad:pad + y0.numel()].view_as(y0)
        fin = fbuf[pad:pad + fin0.numel()].view_as(fin0)
        so = sbuf[pad:pad + so0.numel()].view_as(so0)
        y.copy_(y0)
        so.copy_(so0)
        ssd.ssd_state_correction(y, dev["dt"], dev["A"], dev["C"], dev["init_state"], shard_final=fin0,
                                 final_state=fin, state_out_idx=dev["state_out_idx"], state_out=so)
        torch.cuda.synchronize()
        for buf in (ybuf, fbuf, sbuf):
            assert torch.isnan(buf[:pad].float()).all() and torch.isnan(buf[-pad:].float()).all()
        assert not torch.isnan(y.float()).any() and not torch.isnan(fin).any() and not torch.isnan(so).any()
        outs.append((y.view(torch.int16).cpu(), fin.cpu(), so.cpu()))
    for o in outs[1:]:
        for a, c in zip(outs[0], o):
            assert torch.equal(a, c)
