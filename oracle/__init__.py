"""TEST INFRASTRUCTURE -- the fp64 CPU oracle for the SSD chunked-scan forward.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP path (the library under
``mamba_ssd_scan_06_amd``) and never imports it; the two meet only in the
seeded input generator, which holds none of the scan's arithmetic.

Contents
--------
``ssd_forward``   the token-by-token recurrence in fp64 (plain C, OpenMP over
                  independent rows), see ``ssd_oracle.c`` for the definition
                  and its sources on the pages.
``chunk_cumsum``  the chunk-local cumulative log-decay the block
                  decomposition needs ("Transformers are SSMs" article on
                  cloud.tencent.com.cn, section "SSD算法", yellow part: the
                  scan over chunks runs on modified A factors; the factor of
                  chunk c is exp of the last entry).  Plain definition:
                  cs[b,h,c,i] = A[h] * sum_{k=0..i} dt[b, c*Q+k, h], tokens
                  past the end of the sequence counting as dt = 0.

Every function here is pinned by the ``-m "not gpu"`` tests against closed
forms, brute force and invariants that do not reuse its code.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

GCC_CMD = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", _LIB, "-lm"]


def build(force: bool = False) -> str:
    """Compile ssd_oracle.c with gcc (portable flags: no -march, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        subprocess.run(GCC_CMD, check=True)
    return _LIB


def bind(path: str):
    """Load a compiled oracle library from `path` and declare its signatures."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.oracle_ssd_forward.restype = ctypes.c_int
    lib.oracle_ssd_forward.argtypes = [i64] * 6 + [dp] * 7 + [ctypes.POINTER(ctypes.c_int32)] \
        + [dp] * 3 + [i64, dp, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = bind(_LIB)
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, ctype=ctypes.c_double):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctype))


def ssd_forward(x, dt, A, B, C, D=None, init_state=None, state_out_idx=None,
                chunk: int = 0, nthreads: int = 0, lib=None):
    """Run the fp64 recurrence.

    Shapes: x [b,T,H,P], dt [b,T,H], A [H], B/C [b,T,G,N], D [H] or None,
    init_state [b,H,P,N] or None, state_out_idx [b] int32 or None.
    Returns (y, final_state, state_out or None, chunk_states or None); all fp64.
    `lib` selects another compiled copy of the oracle (see `bind`).
    chunk_states[b,c,h] is the state entering chunk c (recorded when chunk > 0).
    """
    x, dt, A, B, C = (_f64(a) for a in (x, dt, A, B, C))
    D, h0 = _f64(D), _f64(init_state)
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if dt.shape != (b, T, H) or A.shape != (H,) or B.shape != (b, T, G, N) or C.shape != B.shape:
        raise ValueError("oracle: inconsistent shapes")
    if D is not None and D.shape != (H,):
        raise ValueError("oracle: D must be [H]")
    if h0 is not None and h0.shape != (b, H, P, N):
        raise ValueError("oracle: init_state must be [b,H,P,N]")
    idx = None
    if state_out_idx is not None:
        idx = np.ascontiguousarray(state_out_idx, dtype=np.int32)
        if idx.shape != (b,):
            raise ValueError("oracle: state_out_idx must be [b]")
    y = np.empty((b, T, H, P), np.float64)
    fin = np.empty((b, H, P, N), np.float64)
    sout = np.empty((b, H, P, N), np.float64) if idx is not None else None
    nc = (T + chunk - 1) // chunk if chunk > 0 else 0
    cst = np.empty((b, nc, H, P, N), np.float64) if chunk > 0 else None
    rc = (lib or _load()).oracle_ssd_forward(b, T, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                    _ptr(D), _ptr(h0), _ptr(idx, ctypes.c_int32), _ptr(y), _ptr(fin),
                                    _ptr(sout), chunk, _ptr(cst), nthreads)
    if rc != 0:
        raise ValueError(f"oracle_ssd_forward failed with code {rc}")
    return y, fin, sout, cst


def chunk_cumsum(dt, A, chunk: int):
    """cs[b,h,c,i] = A[h] * sum_{k=0..i} dt[b, c*chunk+k, h] in fp64 (dt = 0 past T)."""
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    b, T, H = dt.shape
    nc = (T + chunk - 1) // chunk
    padded = np.zeros((b, nc * chunk, H), np.float64)
    padded[:, :T] = dt
    per_chunk = padded.reshape(b, nc, chunk, H)
    cs = np.cumsum(per_chunk, axis=2) * A[None, None, None, :]
    return np.ascontiguousarray(cs.transpose(0, 3, 1, 2))     # [b, H, nc, chunk]
