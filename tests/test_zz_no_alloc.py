"""The entry point that allocates nothing (ssd_chunk_scan_fwd_noalloc)
against ssd_chunk_scan_fwd: the same kernels on the library's static device
scratch instead of a caller's workspace.  Two calls in a row, the second
smaller, so the second runs on the scratch the first left behind."""
import numpy as np
import pytest
import torch

import mamba_ssd_scan_06_amd as ssd
import ssd_inputs
from ssd_testing import TOL, device_inputs, oracle_run, relerr, to_np, workload

pytestmark = pytest.mark.gpu


def _outputs(dev, b, H, P, N, with_sout):
    y = torch.empty_like(dev["x"])
    fin = torch.empty((b, H, P, N), dtype=torch.float32, device="cuda")
    sout = torch.empty_like(fin) if with_sout else None
    return y, fin, sout


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry(order):
    cases = [
        # b, T, H, P, N, G, Q: both take the chunk-parallel path (fewer than 64 items)
        workload("noalloc_a", 2, 700, 8, 64, 128, 2, 128, "bf16", init_state=True, state_out=True, seed=301),
        workload("noalloc_b", 1, 300, 4, 32, 64, 1, 64, "bf16", init_state=False, state_out=True, seed=302),
    ]
    for wl in cases:
        print(f"\n[case] noalloc {wl}", flush=True)
        shape = ssd.make_shape(wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups)
        need = ssd.ssd_workspace_bytes(shape, wl.chunk, ssd.SSD_DTYPE_BF16)
        assert 0 < need <= ssd.SSD_NOALLOC_SCRATCH_BYTES
        inp = ssd_inputs.generate(wl)
        dev = device_inputs(inp)
        b, H, P, N = wl.batch, wl.nheads, wl.headdim, wl.dstate
        args = (dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], dev["init_state"], wl.chunk,
                dev["state_out_idx"])
        y0, f0, s0 = _outputs(dev, b, H, P, N, True)
        ssd.ssd_chunk_scan_fwd(*args, y=y0, final_state=f0, state_out=s0)
        y1, f1, s1 = _outputs(dev, b, H, P, N, True)
        ssd.ssd_chunk_scan_fwd_noalloc(*args, y=y1, final_state=f1, state_out=s1)
        torch.cuda.synchronize()
        # Same kernels, same inputs: the same bits.
        for name, a, c in (("y", y0, y1), ("final_state", f0, f1), ("state_out", s0, s1)):
            assert torch.equal(a, c), f"{name}: no-alloc entry differs from the workspace entry"
        ref = oracle_run(inp)
        for name, got, key in (("y", y1, "y"), ("final_state", f1, "final"), ("state_out", s1, "state_out")):
            e = relerr(to_np(got), ref[key])
            print(f"  {name}: max rel err {e:.3e}", flush=True)
            assert e <= TOL["bf16"]


def test_noalloc_rejects_calls_beyond_the_scratch():
    # 16 sequences of 4096 tokens, 8 heads of headdim 128 and dstate 256 (16
    # items: the chunk-parallel path) need far more than 64 MiB of workspace.
    b, T, H, P, N, G = 16, 4096, 8, 128, 256, 1
    shape = ssd.make_shape(b, T, H, P, N, G)
    assert ssd.ssd_workspace_bytes(shape, 256, ssd.SSD_DTYPE_BF16) > ssd.SSD_NOALLOC_SCRATCH_BYTES
    x = torch.zeros(b, T, H, P, dtype=torch.bfloat16, device="cuda")
    B = torch.zeros(b, T, G, N, dtype=torch.bfloat16, device="cuda")
    dt = torch.zeros(b, T, H, device="cuda")
    A = -torch.ones(H, device="cuda")
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_chunk_scan_fwd_noalloc(x, dt, A, B, B, None, None, 256)
    assert e.value.name == "SSD_ERR_WORKSPACE"
