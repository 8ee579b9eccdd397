"""Seeded synthetic inputs for the SSD chunked-scan forward.

This module draws random numbers and nothing else: it holds none of the
scan's arithmetic.  Both the HIP path and the fp64 CPU oracle receive the
arrays it returns, and nothing here depends on either of them.

Generator
---------
Counter-based, so any element can be recomputed from (seed, tensor id, index)
alone and the stream does not depend on numpy or torch versions:

* ``splitmix64``: the k-th output of Steele, Lea and Flood's SplitMix64
  ("Fast splittable pseudorandom number generators", OOPSLA 2014) started
  from state ``key``: ``z = key + (k+1)*0x9E3779B97F4A7C15`` followed by the
  published finaliser (xor-shift 30, multiply 0xBF58476D1CE4E5B9, xor-shift
  27, multiply 0x94D049BB133111EB, xor-shift 31).
* ``key = splitmix64_mix(seed * 0x100000001B3 + tensor_id)``.
* uniform(0,1) = ((u >> 11) + 0.5) * 2**-53, never 0 or 1.
* normal = Box-Muller in fp64 from the uniforms at counters 2k and 2k+1.

Draws are made in fp64, rounded to fp32 (round to nearest even), and for
bf16 tensors rounded once more to bf16 (round to nearest even).  The bf16
tensors are returned as their fp32 values (exactly representable) and as raw
uint16 bit patterns.

Value distributions (the five workloads' recipe)
------------------------------------------------
x ~ N(0,1); B, C ~ N(0,1)/sqrt(N); dt = softplus(z + inv_softplus(u_h)) with
z ~ N(0,1) per (b,t,h) and u_h = exp(U(ln 1e-3, ln 1e-1)) per head, where
inv_softplus(u) = ln(expm1(u)); A_h = -exp(U(ln 1, ln 16)); D_h ~ N(0,1);
h0 ~ N(0, 0.1^2) (0.1 is the standard deviation); accepted index
j_b ~ U{0..T-1}.
"""
from __future__ import annotations

import hashlib
import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_BLOCK = 1 << 22  # elements per generation block (bounds temporary memory)

# Tensor ids: part of the counter key, so tensors never share a stream.
TID_X, TID_B, TID_C, TID_DTZ, TID_DTU, TID_A, TID_D, TID_H0, TID_IDX = range(1, 10)


def _mix(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * _M1
    z = z ^ (z >> np.uint64(27))
    z = z * _M2
    return z ^ (z >> np.uint64(31))


def _key(seed: int, tid: int) -> np.uint64:
    with np.errstate(over="ignore"):
        k = np.array([(seed * 0x100000001B3 + tid) & 0xFFFFFFFFFFFFFFFF], dtype=np.uint64)
        return _mix(k)[0]


def _splitmix(key: np.uint64, start: int, count: int) -> np.ndarray:
    ctr = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return _mix(key + ctr * _GOLDEN)


def _to_unit(u: np.ndarray) -> np.ndarray:
    return ((u >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def uniform(seed: int, tid: int, n: int) -> np.ndarray:
    """n fp64 uniforms in (0,1) for tensor `tid`."""
    key = _key(seed, tid)
    return _to_unit(_splitmix(key, 0, n))


def _normal_block(key: np.uint64, start: int, count: int) -> np.ndarray:
    u = _to_unit(_splitmix(key, 2 * start, 2 * count))
    u1, u2 = u[0::2], u[1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def normal(seed: int, tid: int, n: int, workers: int = 8) -> np.ndarray:
    """n fp64 standard normals for tensor `tid` (Box-Muller, counters 2k, 2k+1)."""
    key = _key(seed, tid)
    out = np.empty(n, dtype=np.float64)
    starts = list(range(0, n, _BLOCK))

    def fill(s: int) -> None:
        c = min(_BLOCK, n - s)
        out[s:s + c] = _normal_block(key, s, c)

    if len(starts) <= 1:
        for s in starts:
            fill(s)
    else:
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill, starts))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16, nearest even; returns uint16 bit patterns."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = bits + np.uint32(0x7FFF) + ((bits >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Workload:
    """Problem sizes and dtype of one SSD forward call."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str = "bf16"            # dtype of x, B, C and y: "bf16" or "f32"
    init_state: bool = False       # draw h0 ~ N(0, 0.1^2)
    state_out: bool = False        # draw per-sequence accepted index j_b
    seed: int = 0

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


# The five workloads (seed = 1000 + index).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 256, 2, 16, 16, 1, 64, "f32", seed=1000),
    "mamba2_2.7b": Workload("mamba2_2.7b", 8, 2048, 80, 64, 128, 1, 256, "bf16", seed=1001),
    "long_16k_n256": Workload("long_16k_n256", 1, 16384, 64, 64, 256, 1, 256, "bf16", seed=1002),
    "llama3_8b_hybrid": Workload("llama3_8b_hybrid", 4, 4096, 32, 128, 128, 8, 128, "bf16", seed=1003),
    "spec_verify_k8": Workload("spec_verify_k8", 64, 8, 32, 128, 128, 8, 8, "bf16",
                               init_state=True, state_out=True, seed=1004),
}
WORKLOAD_ORDER = ["tiny_f32", "mamba2_2.7b", "long_16k_n256", "llama3_8b_hybrid", "spec_verify_k8"]


@dataclass
class Inputs:
    """One set of inputs.  Float arrays are fp32 values (bf16-exact where the
    workload is bf16); `*_bits` hold the bf16 bit patterns of x, B, C."""
    wl: Workload
    x: np.ndarray
    dt: np.ndarray
    A: np.ndarray
    B: np.ndarray
    C: np.ndarray
    D: np.ndarray
    init_state: np.ndarray | None
    state_out_idx: np.ndarray | None
    x_bits: np.ndarray | None = None
    B_bits: np.ndarray | None = None
    C_bits: np.ndarray | None = None
    sha256: dict = field(default_factory=dict)


def _softplus(v: np.ndarray) -> np.ndarray:
    return np.where(v > 20.0, v, np.log1p(np.exp(np.minimum(v, 20.0))))


def generate(wl: Workload, seed: int | None = None, workers: int = 8) -> Inputs:
    """Draw all inputs of `wl` (seed defaults to the workload's own)."""
    s = wl.seed if seed is None else seed
    b, T, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups

    def draw_normal(tid: int, shape, scale: float = 1.0) -> np.ndarray:
        n = int(np.prod(shape))
        v = normal(s, tid, n, workers)
        if scale != 1.0:
            v *= scale
        return v.astype(np.float32).reshape(shape)

    x = draw_normal(TID_X, (b, T, H, P))
    Bm = draw_normal(TID_B, (b, T, G, N), 1.0 / math.sqrt(N))
    Cm = draw_normal(TID_C, (b, T, G, N), 1.0 / math.sqrt(N))

    u_h = np.exp(math.log(1e-3) + (math.log(1e-1) - math.log(1e-3)) * uniform(s, TID_DTU, H))
    bias = np.log(np.expm1(u_h))                                   # inv_softplus(u_h)
    z = normal(s, TID_DTZ, b * T * H, workers).reshape(b, T, H)
    dt = _softplus(z + bias[None, None, :]).astype(np.float32)

    A = (-np.exp(math.log(16.0) * uniform(s, TID_A, H))).astype(np.float32)
    D = normal(s, TID_D, H).astype(np.float32)

    h0 = draw_normal(TID_H0, (b, H, P, N), 0.1) if wl.init_state else None
    idx = None
    if wl.state_out:
        idx = np.minimum((uniform(s, TID_IDX, b) * T).astype(np.int64), T - 1).astype(np.int32)

    inp = Inputs(wl, x, dt, A, Bm, Cm, D, h0, idx)
    if wl.dtype == "bf16":
        for name in ("x", "B", "C"):
            bits = f32_to_bf16_bits(getattr(inp, name))
            setattr(inp, name + "_bits", bits)
            setattr(inp, name, bf16_bits_to_f32(bits))
    elif wl.dtype != "f32":
        raise ValueError(f"unknown dtype {wl.dtype}")
    inp.sha256 = digests(inp)
    return inp


def digests(inp: Inputs) -> dict:
    """SHA-256 of every input tensor as handed to the GPU (bf16 bits for bf16)."""
    out = {}
    for name in ("x", "B", "C"):
        bits = getattr(inp, name + "_bits")
        arr = bits if bits is not None else getattr(inp, name)
        out[name] = hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()
    for name in ("dt", "A", "D", "init_state", "state_out_idx"):
        arr = getattr(inp, name)
        if arr is not None:
            out[name] = hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()
    return out
