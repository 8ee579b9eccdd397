"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Every case prints its name, shape and seed first."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_06_amd as ssd
import oracle
import ssd_inputs
from ssd_testing import TOL, device_inputs, gpu_run, kernel_names, oracle_run, relerr, workload

pytestmark = pytest.mark.gpu


def announce(msg):
    print(f"\n[case] {msg}", flush=True)


def check(name, got, ref, tol):
    e = relerr(got, ref)
    print(f"  {name}: max rel err {e:.3e} (tol {tol:.0e})", flush=True)
    assert e <= tol, f"{name}: {e:.3e} > {tol:.0e}"
    return e


@pytest.fixture(scope="module", autouse=True)
def library_loaded():
    # No fallback exists: the HIP library must be there on a GPU machine.
    assert torch.cuda.is_available()
    assert ssd.ssd_abi_version() == 8


# ----------------------------------------------------------- full workloads
@pytest.mark.parametrize("name", ssd_inputs.WORKLOAD_ORDER)
def test_workload_full_size(name):
    wl = ssd_inputs.WORKLOADS[name]
    announce(f"{name} b={wl.batch} T={wl.seqlen} H={wl.nheads} P={wl.headdim} N={wl.dstate} "
             f"G={wl.ngroups} Q={wl.chunk} {wl.dtype} seed={wl.seed}")
    inp = ssd_inputs.generate(wl)
    tol = TOL[wl.dtype]
    ref = oracle_run(inp)
    dev = device_inputs(inp)
    got = gpu_run(inp, dev=dev)
    check("y", got["y"], ref["y"], tol)
    check("final_state", got["final"], ref["final"], tol)
    if wl.state_out:
        check("state_out", got["state_out"], ref["state_out"], tol)
    # Without the D skip, so that D*x cannot hide an error in the scan itself.
    got_nod = gpu_run(inp, dev=dev, use_D=False)
    ref_nod = ref["y"] - inp.D[None, None, :, None].astype(np.float64) * inp.x.astype(np.float64)
    check("y (D = None)", got_nod["y"], ref_nod, tol)


# -------------------------------------------------- individual steps (a1-a6)
STEP_CASES = [
    workload("steps_bf16", 2, 700, 6, 64, 128, 2, 128, "bf16", init_state=True, seed=31),
    workload("steps_f32", 2, 300, 4, 32, 64, 1, 64, "f32", init_state=True, seed=32),
    workload("steps_n256", 1, 600, 4, 64, 256, 1, 256, "bf16", seed=33),
]


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_step_chunk_cumsum(wl):
    # The chunk-local log-decay and the two tables derived from it, element by
    # element against their definitions on the oracle's fp64 sums.
    announce(f"chunk cumsum {wl}")
    inp = ssd_inputs.generate(wl)
    got = gpu_run(inp, return_workspace=True)
    ref = oracle.chunk_cumsum(inp.dt, inp.A, wl.chunk)              # [b,H,nc,Q]
    err = np.max(np.abs(got["cs"] - ref) / np.maximum(np.abs(ref), 1.0))
    print(f"  cs: max err {err:.3e}")
    assert err <= 2e-6
    b, H, nc, Q = ref.shape
    T = wl.seqlen
    dt = np.zeros((b, nc * Q, H))
    dt[:, :T] = inp.dt
    dt = dt.reshape(b, nc, Q, H).transpose(0, 3, 1, 2)             # [b,H,nc,Q]
    t = np.arange(nc * Q).reshape(nc, Q)
    valid = t < T
    # ct = cs log2(e) - log2(dt), +inf past the sequence.
    with np.errstate(divide="ignore"):
        ct_ref = np.where(valid, ref * np.log2(np.e) - np.log2(dt), np.inf)
    assert np.array_equal(np.isinf(got["ct"]), np.isinf(ct_ref)), "ct: +inf entries differ"
    fin = np.isfinite(ct_ref)
    err = np.max(np.abs(got["ct"][fin] - ct_ref[fin]) / np.maximum(np.abs(ct_ref[fin]), 1.0))
    print(f"  ct: max err {err:.3e}")
    assert err <= 4e-6
    # dte = dt_i exp(cs_e - cs_i), e = last token within the sequence of i's 32-token block.
    e = np.minimum((t // 32) * 32 + 31, T - 1)
    cs_e = np.take_along_axis(ref.reshape(b, H, nc * Q), e.reshape(1, 1, -1), axis=2).reshape(ref.shape)
    dte_ref = np.where(valid, dt * np.exp(cs_e - ref), 0.0)
    err = np.max(np.abs(got["dte"] - dte_ref) / np.maximum(np.abs(dte_ref), 1e-30))
    print(f"  dte: max rel err {err:.3e}")
    assert err <= 2e-5


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_step_chunk_states_and_passing(wl):
    # After a chunk-parallel call the workspace holds each chunk's state from
    # a zero start (green) and the state entering each chunk (yellow, the scan
    # over chunks).
    announce(f"chunk states {wl}")
    inp = ssd_inputs.generate(wl)
    got = gpu_run(inp, return_workspace=True)
    ref = oracle_run(inp, chunk=wl.chunk)
    Q, T = wl.chunk, wl.seqlen
    zero_start = []
    for t0 in range(0, T, Q):
        sl = slice(t0, min(t0 + Q, T))
        _, fin, _, _ = oracle.ssd_forward(inp.x[:, sl], inp.dt[:, sl], inp.A, inp.B[:, sl], inp.C[:, sl])
        zero_start.append(fin)
    check("chunk states from a zero start", got["states"], np.stack(zero_start, axis=1), TOL[wl.dtype])
    first = 0 if wl.init_state else 1  # entry 0 is written only with an initial state
    check("states entering each chunk", got["prev"], ref["chunk_states"][:, first:], TOL[wl.dtype])
    check("final_state", got["final"], ref["final"], TOL[wl.dtype])


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_step_single_chunk_state(wl):
    # One chunk, zero initial state: final_state is exactly that chunk's state.
    w1 = workload(wl.name + "_one", wl.batch, wl.chunk - 3, wl.nheads, wl.headdim, wl.dstate, wl.ngroups,
                  wl.chunk, wl.dtype, seed=wl.seed + 1)
    announce(f"single chunk state {w1}")
    inp = ssd_inputs.generate(w1)
    check("chunk state", gpu_run(inp)["final"], oracle_run(inp)["final"], TOL[wl.dtype])


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_step_intra_chunk_only(wl):
    # One chunk, zero initial state, no D: y is the diagonal block alone.
    w1 = workload(wl.name + "_diag", wl.batch, wl.chunk, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.chunk,
                  wl.dtype, seed=wl.seed + 2)
    announce(f"intra-chunk only {w1}")
    inp = ssd_inputs.generate(w1)
    check("y diagonal block", gpu_run(inp, use_D=False)["y"], oracle_run(inp, use_D=False)["y"], TOL[wl.dtype])


@pytest.mark.parametrize("wl", STEP_CASES, ids=lambda w: w.name)
def test_step_state_to_output_only(wl):
    # x = 0 with an initial state: y is the state-to-output term alone.
    w1 = workload(wl.name + "_blue", wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups, wl.chunk,
                  wl.dtype, init_state=True, seed=wl.seed + 3)
    announce(f"state-to-output only {w1}")
    inp = ssd_inputs.generate(w1)
    inp.x = np.zeros_like(inp.x)
    if inp.x_bits is not None:
        inp.x_bits = np.zeros_like(inp.x_bits)
    got, ref = gpu_run(inp), oracle_run(inp)
    check("y from the initial state", got["y"], ref["y"], TOL[wl.dtype])
    check("final_state (pure decay)", got["final"], ref["final"], TOL[wl.dtype])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_state_at_index(dtype):
    T, Q = 150, 32
    wl = workload("at_index_" + dtype, 8, T, 4, 32, 32, 2, Q, dtype, init_state=True, state_out=True, seed=41)
    announce(f"state at index {wl}")
    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp)
    for idx in ([-1, 0, 1, 31, 32, 33, 100, T - 1], [T - 1, 63, 64, 65, 5, 127, 128, 149]):
        inp.state_out_idx = np.array(idx, np.int32)
        dev["state_out_idx"] = torch.from_numpy(inp.state_out_idx).cuda()
        got, ref = gpu_run(inp, dev=dev), oracle_run(inp)
        check(f"state_out {idx}", got["state_out"], ref["state_out"], TOL[dtype])
        check("final_state", got["final"], ref["final"], TOL[dtype])


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chunk_size_invariance(dtype):
    wl = workload("chunk_inv_" + dtype, 2, 300, 4, 64, 64, 2, 64, dtype, init_state=True, seed=51)
    announce(f"chunk-size invariance {wl}")
    inp = ssd_inputs.generate(wl)
    ref = oracle_run(inp)
    dev = device_inputs(inp)
    ys = {}
    for Q in (8, 16, 32, 64, 128, 256):
        got = gpu_run(inp, chunk=Q, dev=dev)
        check(f"Q={Q} y", got["y"], ref["y"], TOL[dtype])
        check(f"Q={Q} final", got["final"], ref["final"], TOL[dtype])
        ys[Q] = got["y"]
    for Q in ys:
        assert relerr(ys[Q], ys[64]) <= 2 * TOL[dtype]


@pytest.mark.parametrize("m", [64, 100, 1])
def test_two_halves(m):
    wl = workload("halves", 2, 257, 4, 64, 128, 1, 64, "bf16", init_state=True, seed=61)
    announce(f"two halves m={m} {wl}")
    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp)
    full = gpu_run(inp, dev=dev)
    ref = oracle_run(inp)
    first = {k: (v[:, :m].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in dev.items()}
    second = {k: (v[:, m:].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in dev.items()}
    y1, f1, _ = ssd.ssd_chunk_scan_fwd(first["x"], first["dt"], first["A"], first["B"], first["C"], first["D"],
                                       first["init_state"], 64)
    y2, f2, _ = ssd.ssd_chunk_scan_fwd(second["x"], second["dt"], second["A"], second["B"], second["C"],
                                       second["D"], f1, 64)
    torch.cuda.synchronize()
    y = torch.cat([y1, y2], dim=1).float().cpu().numpy()
    check("halves y vs oracle", y, ref["y"], 2e-2)
    check("halves final vs oracle", f2.cpu().numpy(), ref["final"], 2e-2)
    check("halves y vs one call", y, full["y"], 2e-2)


# One case per path: chunk-parallel (32 items), single pass (128 items, split
# into block ranges) and one_chunk (8 tokens).
PATH_CASES = [
    ("chunk_parallel", (2, 1000, 8, 128, 128, 2, 128), ssd.SSD_PATH_CHUNK_PARALLEL),
    ("single_pass", (2, 1000, 64, 64, 128, 1, 256), ssd.SSD_PATH_SINGLE_PASS),
    ("one_chunk", (8, 8, 32, 128, 128, 8, 64), ssd.SSD_PATH_ONE_CHUNK),
]


@pytest.mark.parametrize("case", PATH_CASES, ids=lambda c: c[0])
def test_determinism(case):
    name, (b, T, H, P, N, G, Q), path = case
    wl = workload("determinism_" + name, b, T, H, P, N, G, Q, "bf16", init_state=True, state_out=True, seed=71)
    announce(f"determinism {wl} path={name}")
    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp)
    assert ssd.ssd_select_path(ssd.make_shape(b, T, H, P, N, G), Q, ssd.SSD_DTYPE_BF16) == path
    runs = [gpu_run(inp, dev=dev) for _ in range(3)]
    for r in runs[1:]:
        for k in ("y", "final", "state_out"):
            assert np.array_equal(r[k], runs[0][k]), f"{k} differs between identical calls"
    ref = oracle_run(inp)
    check("y", runs[0]["y"], ref["y"], TOL["bf16"])


@pytest.mark.parametrize("case", PATH_CASES, ids=lambda c: c[0])
def test_guard_canaries(case):
    # Outputs inside NaN-filled guard regions: nothing is written outside them
    # and every element inside is written.
    name, (b, T, H, P, N, G, Q), path = case
    wl = workload("canaries_" + name, b, T, H, P, N, G, Q, "bf16", init_state=True, state_out=True, seed=81)
    announce(f"canaries {wl} path={name}")
    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp)
    pad = 4096

    def guarded(n, dtype):
        buf = torch.full((n + 2 * pad,), float("nan"), dtype=dtype, device="cuda")
        return buf, buf[pad:pad + n]

    ybuf, y = guarded(dev["x"].numel(), torch.bfloat16)
    fbuf, fin = guarded(b * H * P * N, torch.float32)
    sbuf, sout = guarded(b * H * P * N, torch.float32)
    outs = dict(y=y.view(dev["x"].shape), final_state=fin.view(b, H, P, N), state_out=sout.view(b, H, P, N))
    got = gpu_run(inp, dev=dev, path=path, outputs=outs)
    for buf in (ybuf, fbuf, sbuf):
        assert torch.isnan(buf[:pad].float()).all() and torch.isnan(buf[-pad:].float()).all(), "write outside output"
        assert torch.isfinite(buf[pad:-pad].float()).all(), "output not fully written"
    ref = oracle_run(inp)
    for k in ("y", "final", "state_out"):
        check(k, got[k], ref[k], TOL["bf16"])


# ---------------------------------------------------------------- edge cases
EDGE = [
    # b, T, H, P, N, G, Q, dtype
    (1, 1, 1, 16, 16, 1, 8, "f32"),
    (3, 7, 2, 16, 32, 2, 8, "bf16"),
    (2, 33, 4, 32, 64, 4, 32, "bf16"),
    (1, 257, 2, 64, 256, 1, 256, "bf16"),
    (2, 255, 8, 128, 256, 2, 128, "bf16"),
    (1, 129, 3, 128, 16, 3, 16, "bf16"),
    (2, 100, 4, 64, 128, 1, 256, "f32"),
    (1, 1000, 2, 16, 16, 2, 64, "f32"),
    (4, 9, 32, 128, 128, 8, 8, "bf16"),
    (1, 64, 1, 64, 64, 1, 64, "bf16"),
]


@pytest.mark.parametrize("case", EDGE, ids=lambda c: "b{}_T{}_H{}_P{}_N{}_G{}_Q{}_{}".format(*c))
def test_edge_shapes(case):
    b, T, H, P, N, G, Q, dtype = case
    wl = workload("edge", b, T, H, P, N, G, Q, dtype, init_state=True, state_out=True, seed=91 + T)
    announce(f"edge {wl}")
    inp = ssd_inputs.generate(wl)
    got, ref = gpu_run(inp), oracle_run(inp)
    for k in ("y", "final", "state_out"):
        check(k, got[k], ref[k], TOL[dtype])


# Calls that fit one chunk of at most 32 tokens take the fused one-kernel
# path (the multi-step verify); the shapes below cover T = 1, T < Q, T = Q =
# 32, N = 256, fp32, no initial state and no D.
ONE_CHUNK = [
    # b, T, H, P, N, G, Q, dtype, init_state
    (2, 1, 4, 64, 128, 1, 8, "bf16", True),
    (3, 5, 6, 128, 64, 3, 8, "bf16", True),
    (2, 32, 4, 64, 256, 2, 32, "bf16", True),
    (2, 31, 2, 32, 64, 1, 64, "f32", True),
    (2, 8, 4, 128, 128, 4, 16, "bf16", False),
]


@pytest.mark.parametrize("case", ONE_CHUNK, ids=lambda c: "b{}_T{}_H{}_P{}_N{}_G{}_Q{}_{}_init{}".format(*c))
def test_one_chunk_fused(case):
    b, T, H, P, N, G, Q, dtype, init = case
    wl = workload("one_chunk", b, T, H, P, N, G, Q, dtype, init_state=init, state_out=True, seed=131 + T)
    announce(f"one chunk {wl}")
    inp = ssd_inputs.generate(wl)
    got, ref = gpu_run(inp), oracle_run(inp)
    for k in ("y", "final", "state_out"):
        check(k, got[k], ref[k], TOL[dtype])
    got0, ref0 = gpu_run(inp, use_D=False), oracle_run(inp, use_D=False)
    check("y without D", got0["y"], ref0["y"], TOL[dtype])


def test_decode_in_place():
    # Three single-token steps that update the state in place (final_state is
    # init_state) equal one call over the three tokens.
    wl = workload("decode", 16, 3, 8, 64, 128, 2, 64, "bf16", init_state=True, seed=141)
    announce(f"decode in place {wl}")
    inp = ssd_inputs.generate(wl)
    ref = oracle_run(inp)
    dev = device_inputs(inp)
    h = dev["init_state"].clone()
    ys = []
    for t in range(wl.seqlen):
        sl = slice(t, t + 1)
        y, fin, _ = ssd.ssd_chunk_scan_fwd(dev["x"][:, sl].contiguous(), dev["dt"][:, sl].contiguous(), dev["A"],
                                           dev["B"][:, sl].contiguous(), dev["C"][:, sl].contiguous(), dev["D"],
                                           h, 64, final_state=h)
        assert fin.data_ptr() == h.data_ptr()
        ys.append(y)
    torch.cuda.synchronize()
    y_all = torch.cat(ys, dim=1).float().cpu().numpy()
    check("y", y_all, ref["y"], 2e-2)
    check("state", h.cpu().numpy(), ref["final"], 2e-2)


@pytest.mark.parametrize("T", [300, 20])
def test_in_place_with_state_out(T):
    # final_state == init_state on the chunked path (T = 300) and the fused
    # one-chunk path (T = 20), with accepted indices including -1.
    wl = workload("inplace", 4, T, 4, 64, 64, 2, 64, "bf16", init_state=True, state_out=True, seed=151 + T)
    announce(f"in place {wl}")
    inp = ssd_inputs.generate(wl)
    idx = np.array([-1, 0, T // 2, T - 1], np.int32)
    ref = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state, idx)
    dev = device_inputs(inp)
    h = dev["init_state"].clone()
    y, fin, sout = ssd.ssd_chunk_scan_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], h, 64,
                                          torch.from_numpy(idx).cuda(), final_state=h)
    torch.cuda.synchronize()
    check("y", y.float().cpu().numpy(), ref[0], 2e-2)
    check("final (in place)", h.cpu().numpy(), ref[1], 2e-2)
    check("state_out", sout.cpu().numpy(), ref[2], 2e-2)


# ------------------------------------------------- single-pass fused forward
# b, T, H, P, N, G, Q, init_state, state_out, D
FUSED = [
    (4, 1800, 80, 64, 128, 1, 256, True, True, True),    # the 2.7B layer's configuration, 8 chunks, last of 8
    (2, 500, 128, 32, 64, 1, 128, True, True, True),     # 4 chunks, last of 116
    (3, 400, 96, 64, 128, 2, 128, False, True, True),    # two groups, zero start, 4 chunks
    (4, 200, 64, 64, 128, 1, 256, True, True, False),    # one partial chunk, no D
    (2, 1024, 128, 64, 64, 4, 256, True, False, True),   # four groups, 4 full chunks
    # Work split over a persistent grid of one workgroup per CU (256 here):
    (2, 300, 200, 64, 64, 1, 128, True, True, True),     # 400 pairs: 144 left over, too many to split
    (3, 700, 96, 64, 128, 1, 256, True, True, True),     # 288 pairs: 32 split in halves of 3 chunks (1 + 2)
    # Many groups: every group's B and C rows are read by few heads.
    (2, 600, 128, 64, 128, 64, 256, True, True, True),   # 2 heads per group
    (2, 700, 128, 32, 64, 32, 128, True, True, True),    # 4 heads per group, 32 groups
    # headdim 128: each head runs as two 64-channel items
    (2, 700, 64, 128, 128, 8, 128, True, True, True),    # 256 items
    (3, 600, 48, 128, 64, 4, 256, True, True, True),     # 288 items: 32 split in chunk halves
    (2, 450, 128, 128, 64, 128, 128, False, True, False),  # 512 items, one head per group, zero start, no D
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: "b{}_T{}_H{}_P{}_N{}_G{}_Q{}_init{}_sout{}_D{}".format(*c))
def test_fused_forward(case):
    b, T, H, P, N, G, Q, init, sout, use_D = case
    wl = workload("fused", b, T, H, P, N, G, Q, "bf16", init_state=init, state_out=sout, seed=211 + T + H)
    announce(f"fused forward {wl} D={use_D}")
    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp)
    names = kernel_names(inp, dev=dev)
    print(f"  kernels: {names}", flush=True)
    assert names == ["chunk_scan_fused"], names
    got, ref = gpu_run(inp, dev=dev, use_D=use_D), oracle_run(inp, use_D=use_D)
    check("y", got["y"], ref["y"], TOL["bf16"])
    check("final_state", got["final"], ref["final"], TOL["bf16"])
    if sout:
        check("state_out", got["state_out"], ref["state_out"], TOL["bf16"])


# Degenerate values through the single pass: dt = 0 tokens (no input, no
# decay; ct = +inf) at the start, inside a block, across a block boundary and
# at the end, and A = 0 heads (no decay at all: the state is a plain sum).
@pytest.mark.parametrize("zero_dt,zero_A", [(True, False), (False, True), (True, True)])
def test_fused_degenerate_values(zero_dt, zero_A):
    b, T, H, P, N, G, Q = 2, 700, 64, 64, 128, 2, 256
    wl = workload("fused_degenerate", b, T, H, P, N, G, Q, "bf16", init_state=True, state_out=True, seed=241)
    announce(f"fused degenerate {wl} dt=0 tokens: {zero_dt} A=0 heads: {zero_A}")
    inp = ssd_inputs.generate(wl)
    if zero_dt:
        for t in (0, 1, 50, 127, 128, 129, 300, 301, 302, T - 1):
            inp.dt[:, t, :] = 0.0
        inp.dt[1, 400:460, 5] = 0.0
    if zero_A:
        inp.A[::3] = 0.0
    inp.state_out_idx = np.array([0, 129], np.int32)
    dev = device_inputs(inp)
    assert kernel_names(inp, dev=dev) == ["chunk_scan_fused"]
    got, ref = gpu_run(inp, dev=dev), oracle_run(inp)
    for k in ("y", "final", "state_out"):
        check(k, got[k], ref[k], TOL["bf16"])


# dstate 256 with at most 64 items (the long-sequence configuration's
# geometry at shorter lengths): these take the chunk-parallel path.
N256 = [
    # b, T, H, P, N, G, Q, init_state, state_out
    (1, 2500, 64, 64, 256, 1, 256, True, True),    # 64 items, 10 chunks, last partial
    (2, 1300, 16, 64, 256, 2, 128, False, True),   # 32 items, zero start
    (1, 777, 8, 128, 256, 1, 256, True, False),    # headdim 128, 8 heads
    (2, 2000, 64, 64, 256, 1, 256, True, True),    # 128 items, 8 chunks: head-batched chunk states, n in halves
]


@pytest.mark.parametrize("case", N256, ids=lambda c: "b{}_T{}_H{}_P{}_N{}_G{}_Q{}_init{}_sout{}".format(*c))
def test_dstate_256(case):
    b, T, H, P, N, G, Q, init, sout = case
    wl = workload("n256", b, T, H, P, N, G, Q, "bf16", init_state=init, state_out=sout, seed=261 + T)
    announce(f"dstate 256 {wl}")
    inp = ssd_inputs.generate(wl)
    got, ref = gpu_run(inp), oracle_run(inp)
    for k in ("y", "final") + (("state_out",) if sout else ()):
        check(k, got[k], ref[k], TOL["bf16"])


def test_paths_agree_at_layer_shape():
    # The 2.7B layer's shape (fewer tokens) through the single pass and the
    # chunk-parallel kernels, each against the oracle.
    wl = workload("paths", 2, 1100, 80, 64, 128, 1, 256, "bf16", init_state=True, state_out=True, seed=251)
    announce(f"both paths {wl}")
    inp = ssd_inputs.generate(wl)
    dev = device_inputs(inp)
    ref = oracle_run(inp)
    for path in (ssd.SSD_PATH_SINGLE_PASS, ssd.SSD_PATH_CHUNK_PARALLEL):
        got = gpu_run(inp, dev=dev, path=path)
        for k in ("y", "final", "state_out"):
            check(f"{ssd.PATH_NAMES[path]} {k}", got[k], ref[k], TOL["bf16"])


def test_fused_in_place():
    # final_state == init_state through the fused kernel, indices incl. -1.
    wl = workload("fused_inplace", 4, 450, 64, 64, 64, 1, 128, "bf16", init_state=True, state_out=True, seed=231)
    announce(f"fused in place {wl}")
    inp = ssd_inputs.generate(wl)
    idx = np.array([-1, 0, 200, 449], np.int32)
    ref = oracle.ssd_forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.init_state, idx)
    dev = device_inputs(inp)
    dev["state_out_idx"] = torch.from_numpy(idx).cuda()
    assert "chunk_scan_fused" in kernel_names(inp, dev=dev)
    h = dev["init_state"].clone()
    y, fin, sout = ssd.ssd_chunk_scan_fwd(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], h, 128,
                                          dev["state_out_idx"], final_state=h)
    torch.cuda.synchronize()
    check("y", y.float().cpu().numpy(), ref[0], 2e-2)
    check("final (in place)", h.cpu().numpy(), ref[1], 2e-2)
    check("state_out", sout.cpu().numpy(), ref[2], 2e-2)


def test_empty_sequence():
    announce("empty sequence T=0")
    h0 = torch.randn(2, 4, 64, 128, device="cuda")
    x = torch.empty(2, 0, 4, 64, dtype=torch.bfloat16, device="cuda")
    B = torch.empty(2, 0, 1, 128, dtype=torch.bfloat16, device="cuda")
    dt = torch.empty(2, 0, 4, device="cuda")
    A = -torch.ones(4, device="cuda")
    idx = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    y, fin, sout = ssd.ssd_chunk_scan_fwd(x, dt, A, B, B, None, h0, 64, idx)
    torch.cuda.synchronize()
    assert y.numel() == 0
    assert torch.equal(fin, h0) and torch.equal(sout, h0)
    _, fin0, _ = ssd.ssd_chunk_scan_fwd(x, dt, A, B, B, None, None, 64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(fin0) == 0


def test_empty_batch():
    announce("empty batch b=0")
    x = torch.empty(0, 16, 4, 64, dtype=torch.bfloat16, device="cuda")
    B = torch.empty(0, 16, 1, 128, dtype=torch.bfloat16, device="cuda")
    y, fin, _ = ssd.ssd_chunk_scan_fwd(x, torch.empty(0, 16, 4, device="cuda"), -torch.ones(4, device="cuda"),
                                       B, B, None, None, 64)
    assert y.numel() == 0 and fin.numel() == 0
