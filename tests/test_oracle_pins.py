"""The fp64 oracle against pins that do not reuse its code (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle.ssd_forward)


def test_oracle_thread_count_invariant():
    rng = np.random.default_rng(3)
    pr = pins.problem(rng, b=2, T=30, H=4, P=5, N=7, G=2)
    y1, f1, _, _ = oracle.ssd_forward(**pr, nthreads=1)
    y4, f4, _, _ = oracle.ssd_forward(**pr, nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(f1, f4)


def test_oracle_rejects_bad_groups():
    rng = np.random.default_rng(4)
    pr = pins.problem(rng, H=4, G=3)
    with pytest.raises(ValueError):
        oracle.ssd_forward(**pr)


def test_chunk_cumsum_constant_dt():
    # dt = delta everywhere: cs[c, i] = A * delta * (i + 1); past T it stays flat.
    b, T, H, Q = 2, 10, 3, 4
    A = np.array([-1.0, -2.5, -0.125])
    cs = oracle.chunk_cumsum(np.full((b, T, H), 0.5), A, Q)
    assert cs.shape == (b, H, 3, Q)
    for h in range(H):
        for c in range(3):
            for i in range(Q):
                valid = min(i, T - 1 - c * Q)
                assert cs[0, h, c, i] == pytest.approx(A[h] * 0.5 * (valid + 1), rel=1e-15)


def test_chunk_cumsum_against_recurrence_decay():
    # exp(cs[b,h,c,i]) is the decay a unit state suffers from the start of chunk c
    # through token c*Q+i; the recurrence with x = 0 and h_init = 1 computes it.
    rng = np.random.default_rng(5)
    b, T, H, Q = 2, 11, 3, 4
    dt = rng.uniform(0.05, 0.9, size=(b, T, H))
    A = -rng.uniform(0.2, 2.0, size=H)
    cs = oracle.chunk_cumsum(dt, A, Q)
    for c in range((T + Q - 1) // Q):
        for i in range(Q):
            t = min(c * Q + i, T - 1)
            n = t - c * Q + 1
            ones = np.ones((b, n, H, 1))
            _, fin, _, _ = oracle.ssd_forward(np.zeros((b, n, H, 1)), dt[:, c * Q:t + 1], A,
                                              np.ones((b, n, 1, 1)), np.ones((b, n, 1, 1)),
                                              init_state=np.ones((b, H, 1, 1)))
            pins.close(np.exp(cs[:, :, c, i]), fin[:, :, 0, 0], what=f"decay c={c} i={i}")
            del ones


def test_golden_scalar_geometric():
    """Hand-worked example stored in tests/golden/scalar_geometric.json."""
    with open(os.path.join(HERE, "golden", "scalar_geometric.json")) as f:
        g = json.load(f)
    T = len(g["y"])
    one = np.ones((1, T, 1, 1))
    y, fin, _, _ = oracle.ssd_forward(one, np.full((1, T, 1), g["dt"]), np.array([g["A"]]), one, one)
    for t in range(T):
        assert y[0, t, 0, 0] == pytest.approx(eval(g["y"][t], {"ln2": math.log(2.0)}), rel=1e-14)


def test_golden_regression():
    """Oracle outputs stored by tests/golden/make_golden.py (calls only oracle/)."""
    import sys
    sys.path.insert(0, os.path.join(HERE, "golden"))
    import make_golden
    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        g = json.load(f)
    y, fin, sout, _ = make_golden.run_case()
    np.testing.assert_allclose(y.ravel(), np.array(g["y"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(fin.ravel(), np.array(g["final_state"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(sout.ravel(), np.array(g["state_out"]), rtol=0, atol=1e-13)
