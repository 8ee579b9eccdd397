"""Pins for the fp64 oracle: checks that do not reuse its code.

Each ``pin_*`` function takes a forward callable with the signature of
``oracle.ssd_forward`` and raises AssertionError when the callable disagrees
with a closed form, a brute-force evaluation, a library routine or an
invariant that the pages fix.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle with a
planted mistake and requires that some pin fails for every mistake.

Sources (the pages' formulas are lost; the recurrence reading is stated in
``oracle/ssd_oracle.c``):
* "Transformers are SSMs" article (cloud.tencent.com.cn), sections
  "研究贡献" and "核心创新——SSD": the SSM forward is a multiplication by a
  semiseparable matrix; linear (recurrent) and quadratic (attention-like)
  forms compute the same thing -> brute force, chunk-size independence.
* same article, sections "SSD算法" and "深入解析分块与状态传递机制": the
  block decomposition is exact and the passed state carries everything
  earlier chunks contribute -> chunked evaluation, two halves.
* "3天把Llama训成Mamba" article (blog.csdn.net), section
  "从 Transformer 到 Mamba": a linear RNN is linear attention with
  x, B, C in the roles of V, K, Q -> A = 0 reduces to causal linear attention.
* same article, section "推测解码": the verifier returns the outputs, the
  state at the last accepted position and the state after the last token ->
  state_out semantics.
* same article, section "模型架构和训练", and the Mamba-2 article's
  grouped-value heads ("研究贡献") -> group sharing.
"""
from __future__ import annotations

import math

import numpy as np

RTOL = 1e-11


def close(got, ref, rtol=RTOL, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    scale = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1e-300)
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= rtol * scale, f"{what}: max abs err {err:.3e} > {rtol:.1e} * {scale:.3e}"


def problem(rng, b=2, T=13, H=4, P=3, N=5, G=2, D=True, h0=True, dt_scale=1.0):
    x = rng.normal(size=(b, T, H, P))
    dt = rng.uniform(0.05, 0.9, size=(b, T, H)) * dt_scale
    A = -rng.uniform(0.2, 2.0, size=H)
    B = rng.normal(size=(b, T, G, N))
    C = rng.normal(size=(b, T, G, N))
    Dv = rng.normal(size=H) if D else None
    h = rng.normal(size=(b, H, P, N)) if h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=Dv, init_state=h)


# ---------------------------------------------------------------- brute force
def brute_force(x, dt, A, B, C, D=None, init_state=None):
    """Materialise the semiseparable matrix M[t,s] = (C_t.B_s) * prod_{k=s+1..t} exp(dt_k A)
    and the decay of the initial state, per (b, h); evaluate y and the final state."""
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    fin = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = h * G // H
            step = np.exp(dt[bi, :, h] * A[h])              # per-token decay factors
            L = np.zeros((T, T))
            for t in range(T):
                for s in range(t + 1):
                    L[t, s] = np.prod(step[s + 1:t + 1])     # empty product = 1
            M = L * (C[bi, :, g, :] @ B[bi, :, g, :].T)
            u = dt[bi, :, h, None] * x[bi, :, h, :]          # [T, P]
            y[bi, :, h, :] = M @ u
            for s in range(T):
                fin[bi, h] += np.prod(step[s + 1:]) * np.outer(u[s], B[bi, s, g])
            if init_state is not None:
                from_init = np.array([np.prod(step[:t + 1]) for t in range(T)])
                y[bi, :, h, :] += from_init[:, None] * (C[bi, :, g, :] @ init_state[bi, h].T)
                fin[bi, h] += np.prod(step) * init_state[bi, h]
            if D is not None:
                y[bi, :, h, :] += D[h] * x[bi, :, h, :]
    return y, fin


def chunked(x, dt, A, B, C, D, init_state, Q):
    """The four-part block decomposition in plain fp64 numpy (test-only):
    diagonal blocks in quadratic form, chunk states, state passing over chunks,
    state-to-output.  Documents the arithmetic the GPU kernels perform."""
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    fin = np.zeros((b, H, P, N))
    for bi in range(b):
        for h in range(H):
            g = h * G // H
            state = np.zeros((P, N)) if init_state is None else init_state[bi, h].copy()
            for c0 in range(0, T, Q):
                sl = slice(c0, min(c0 + Q, T))
                cs = np.cumsum(A[h] * dt[bi, sl, h])                       # chunk-local
                Cc, Bc = C[bi, sl, g, :], B[bi, sl, g, :]
                u = dt[bi, sl, h, None] * x[bi, sl, h, :]
                Lm = np.tril(np.exp(np.tril(cs[:, None] - cs[None, :])))   # mask before exp
                y_diag = (Lm * (Cc @ Bc.T)) @ u                             # orange
                y_off = np.exp(cs)[:, None] * (Cc @ state.T)                # blue
                S = (np.exp(cs[-1] - cs)[:, None] * u).T @ Bc              # green
                state = np.exp(cs[-1]) * state + S                         # yellow
                y[bi, sl, h, :] = y_diag + y_off
            fin[bi, h] = state
            if D is not None:
                y[bi, :, h, :] += D[h] * x[bi, :, h, :]
    return y, fin


# ----------------------------------------------------------------------- pins
def pin_brute_force(fwd):
    rng = np.random.default_rng(11)
    for kw in (dict(), dict(D=False, h0=False), dict(b=1, T=1, H=2, G=1), dict(T=24, H=3, G=3, P=2, N=2)):
        pr = problem(rng, **kw)
        y, fin, _, _ = fwd(**pr)
        yr, fr = brute_force(**pr)
        close(y, yr, what="brute y")
        close(fin, fr, what="brute final")


def pin_scalar_geometric(fwd):
    # H=P=N=1, dt = delta, A = alpha, x = B = C = 1, D = 0:
    # h_t = a^(t+1) h_init + delta (1 - a^(t+1)) / (1 - a), a = exp(delta alpha); y_t = h_t.
    for delta, alpha, hinit, T in ((0.3, -1.5, 0.7, 9), (1.0, -0.25, -2.0, 5), (0.01, -3.0, 0.0, 17)):
        a = math.exp(delta * alpha)
        ref = np.array([a ** (t + 1) * hinit + delta * (1 - a ** (t + 1)) / (1 - a) for t in range(T)])
        one = np.ones((1, T, 1, 1))
        y, fin, _, _ = fwd(one, np.full((1, T, 1), delta), np.array([alpha]), one, one,
                           init_state=np.full((1, 1, 1, 1), hinit))
        close(y[0, :, 0, 0], ref, what="geometric y")
        close(fin[0, 0, 0, 0], ref[-1], what="geometric final")


def pin_linear_attention(fwd):
    # A = 0: no decay, so y = tril(C B^T) (dt * x) + D x, via numpy tril/matmul.
    rng = np.random.default_rng(12)
    pr = problem(rng, h0=False)
    pr["A"] = np.zeros_like(pr["A"])
    y, fin, _, _ = fwd(**pr)
    x, dt, B, C, D = pr["x"], pr["dt"], pr["B"], pr["C"], pr["D"]
    b, T, H, P = x.shape
    G = B.shape[2]
    for bi in range(b):
        for h in range(H):
            g = h * G // H
            u = dt[bi, :, h, None] * x[bi, :, h, :]
            ref = np.tril(C[bi, :, g] @ B[bi, :, g].T) @ u + D[h] * x[bi, :, h]
            close(y[bi, :, h], ref, what="A=0 y")
            close(fin[bi, h], u.T @ B[bi, :, g], what="A=0 final")


def pin_zero_dt(fwd):
    # dt = 0: decay 1 and no input, so h_t = h_init and y_t = C_t h_init^T + D x_t.
    rng = np.random.default_rng(13)
    pr = problem(rng)
    pr["dt"] = np.zeros_like(pr["dt"])
    y, fin, _, _ = fwd(**pr)
    x, C, D, h0 = pr["x"], pr["C"], pr["D"], pr["init_state"]
    H, G = x.shape[2], C.shape[2]
    for h in range(H):
        g = h * G // H
        ref = np.einsum("btn,bpn->btp", C[:, :, g], h0[:, h]) + D[h] * x[:, :, h]
        close(y[:, :, h], ref, what="dt=0 y")
    close(fin, h0, what="dt=0 final")


def pin_zero_x(fwd):
    # x = 0: pure decay of the initial state, h_t = exp(A sum_{k<=t} dt_k) h_init.
    rng = np.random.default_rng(14)
    pr = problem(rng)
    pr["x"] = np.zeros_like(pr["x"])
    y, fin, _, _ = fwd(**pr)
    dt, A, C, h0 = pr["dt"], pr["A"], pr["C"], pr["init_state"]
    H, G = dt.shape[2], C.shape[2]
    for h in range(H):
        g = h * G // H
        decay = np.exp(A[h] * np.cumsum(dt[:, :, h], axis=1))           # [b, T]
        ref = decay[:, :, None] * np.einsum("btn,bpn->btp", C[:, :, g], h0[:, h])
        close(y[:, :, h], ref, what="x=0 y")
        close(fin[:, h], np.exp(A[h] * dt[:, :, h].sum(1))[:, None, None] * h0[:, h], what="x=0 final")


def pin_single_step(fwd):
    # T = 1 from a given state: y = (a h0 + delta x B^T) C + D x with a = exp(delta A).
    rng = np.random.default_rng(15)
    pr = problem(rng, T=1)
    y, fin, _, _ = fwd(**pr)
    x, dt, A, B, C, D, h0 = (pr[k] for k in ("x", "dt", "A", "B", "C", "D", "init_state"))
    b, _, H, P = x.shape
    G = B.shape[2]
    for bi in range(b):
        for h in range(H):
            g = h * G // H
            d = dt[bi, 0, h]
            hn = math.exp(d * A[h]) * h0[bi, h] + d * np.outer(x[bi, 0, h], B[bi, 0, g])
            close(fin[bi, h], hn, what="single-step state")
            close(y[bi, 0, h], hn @ C[bi, 0, g] + D[h] * x[bi, 0, h], what="single-step y")


def pin_chunk_independence(fwd):
    rng = np.random.default_rng(16)
    pr = problem(rng, T=17)
    y, fin, _, _ = fwd(**pr)
    for Q in (1, 3, 8, 16, 17, 32):
        yc, fc = chunked(**pr, Q=Q)
        close(y, yc, what=f"chunked Q={Q} y")
        close(fin, fc, what=f"chunked Q={Q} final")


def pin_two_halves(fwd):
    rng = np.random.default_rng(17)
    pr = problem(rng, T=20)
    y, fin, _, _ = fwd(**pr)
    for m in (1, 8, 13, 19):
        first = {k: (v[:, :m] if k in ("x", "dt", "B", "C") else v) for k, v in pr.items()}
        second = {k: (v[:, m:] if k in ("x", "dt", "B", "C") else v) for k, v in pr.items()}
        y1, f1, _, _ = fwd(**first)
        second["init_state"] = f1
        y2, f2, _, _ = fwd(**second)
        close(np.concatenate([y1, y2], axis=1), y, what=f"two halves m={m} y")
        close(f2, fin, what=f"two halves m={m} final")


def pin_state_out(fwd):
    rng = np.random.default_rng(18)
    pr = problem(rng, b=4, T=9)
    idx = np.array([-1, 0, 5, 8], np.int32)
    y, fin, sout, _ = fwd(**pr, state_out_idx=idx)
    close(sout[0], pr["init_state"][0], what="state_out(-1) = init")
    close(sout[3], fin[3], what="state_out(T-1) = final")
    for bi in (1, 2):
        j = int(idx[bi])
        sub = {k: (v[bi:bi + 1, :j + 1] if k in ("x", "dt", "B", "C") else v) for k, v in pr.items()}
        sub["init_state"] = pr["init_state"][bi:bi + 1]
        _, fj, _, _ = fwd(**sub)
        close(sout[bi], fj[0], what=f"state_out({j}) = state after token {j}")
    y2, _, _, _ = fwd(**pr)
    close(y, y2, rtol=0.0, what="state_out leaves y unchanged")


def pin_linearity(fwd):
    rng = np.random.default_rng(19)
    pr = problem(rng)
    base = dict(pr, init_state=None)
    x1, x2 = pr["x"], rng.normal(size=pr["x"].shape)
    y1, f1, _, _ = fwd(**dict(base, x=x1))
    y2, f2, _, _ = fwd(**dict(base, x=x2))
    y3, f3, _, _ = fwd(**dict(base, x=x1 + 2.0 * x2))
    close(y3, y1 + 2.0 * y2, rtol=1e-10, what="linear in x: y")
    close(f3, f1 + 2.0 * f2, rtol=1e-10, what="linear in x: final")
    yh, fh, _, _ = fwd(**dict(pr, x=np.zeros_like(x1), D=None))
    yall, fall, _, _ = fwd(**pr)
    close(yall, y1 + yh, rtol=1e-10, what="linear in h0: y")
    close(fall, f1 + fh, rtol=1e-10, what="linear in h0: final")


def pin_groups(fwd):
    # G groups == G = H with B and C repeated for the H/G heads of each group.
    rng = np.random.default_rng(20)
    pr = problem(rng, H=6, G=2)
    y, fin, _, _ = fwd(**pr)
    H, G = 6, 2
    rep = np.array([h * G // H for h in range(H)])
    pr2 = dict(pr, B=pr["B"][:, :, rep], C=pr["C"][:, :, rep])
    y2, f2, _, _ = fwd(**pr2)
    close(y, y2, what="groups y")
    close(fin, f2, what="groups final")


def pin_chunk_states(fwd):
    rng = np.random.default_rng(21)
    pr = problem(rng, T=11)
    Q = 4
    _, _, _, cst = fwd(**pr, chunk=Q)
    close(cst[:, 0], pr["init_state"], what="chunk 0 starts from init")
    for c in (1, 2):
        sub = {k: (v[:, :c * Q] if k in ("x", "dt", "B", "C") else v) for k, v in pr.items()}
        _, fc, _, _ = fwd(**sub)
        close(cst[:, c], fc, what=f"state entering chunk {c}")


ALL_PINS = [pin_brute_force, pin_scalar_geometric, pin_linear_attention, pin_zero_dt, pin_zero_x,
            pin_single_step, pin_chunk_independence, pin_two_halves, pin_state_out, pin_linearity,
            pin_groups, pin_chunk_states]
