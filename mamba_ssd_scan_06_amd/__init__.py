"""Python binding of libssd, the MI355X (gfx950) SSD chunked-scan forward.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libssd.so`` (built from ``csrc/`` by ``build.py``).  torch
supplies device memory and the current stream.  The functions carry the
names of the C entry points declared in ``include/ssd.h``; see there for the
operation, layouts, ownership and error behaviour.

There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "SsdError", "ssd_abi_version", "ssd_status_string", "ssd_last_error", "ssd_workspace_bytes",
    "ssd_get_workspace_layout", "ssd_select_path", "ssd_chunk_scan_fwd", "ssd_chunk_scan_fwd_ex",
    "ssd_chunk_scan_fwd_noalloc", "ssd_state_correction", "SSD_NOALLOC_SCRATCH_BYTES", "workspace_views", "library_path", "SSD_PATH_AUTO", "SSD_PATH_ONE_CHUNK", "SSD_PATH_SINGLE_PASS",
    "SSD_PATH_CHUNK_PARALLEL",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libssd.so")
_lib = None

SSD_DTYPE_F32 = 0
SSD_DTYPE_BF16 = 1
SSD_NOALLOC_SCRATCH_BYTES = 64 << 20
SSD_PATH_AUTO = 0
SSD_PATH_ONE_CHUNK = 1
SSD_PATH_SINGLE_PASS = 2
SSD_PATH_CHUNK_PARALLEL = 3
PATH_NAMES = {SSD_PATH_AUTO: "auto", SSD_PATH_ONE_CHUNK: "one_chunk", SSD_PATH_SINGLE_PASS: "single_pass",
              SSD_PATH_CHUNK_PARALLEL: "chunk_parallel"}
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_CHUNK", 4: "SSD_ERR_ALIGN",
          5: "SSD_ERR_WORKSPACE", 6: "SSD_ERR_ALIAS", 7: "SSD_ERR_ARGS", 8: "SSD_ERR_HIP",
          9: "SSD_ERR_UNSUPPORTED"}


class ssd_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64)]


class ssd_workspace_layout(ctypes.Structure):
    _fields_ = [("cumsum_offset", ctypes.c_size_t), ("ct_offset", ctypes.c_size_t),
                ("dt_decay_offset", ctypes.c_size_t), ("states_offset", ctypes.c_size_t),
                ("prev_offset", ctypes.c_size_t), ("hj_offset", ctypes.c_size_t),
                ("total_bytes", ctypes.c_size_t), ("nchunks", ctypes.c_int64)]


class SsdError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m mamba_ssd_scan_06_amd.build`")
    # torch ships its own HIP runtime under the same soname; loading torch
    # first makes libssd bind to that one, so torch's streams and memory are
    # the library's too (one runtime per process).
    import torch  # noqa: F401
    lib = ctypes.CDLL(_LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    shp = ctypes.POINTER(ssd_shape)
    lib.ssd_workspace_bytes.argtypes = [shp, i32, i32]
    lib.ssd_workspace_bytes.restype = sz
    lib.ssd_get_workspace_layout.argtypes = [shp, i32, i32, ctypes.POINTER(ssd_workspace_layout)]
    lib.ssd_get_workspace_layout.restype = i32
    lib.ssd_select_path.argtypes = [shp, i32, i32]
    lib.ssd_select_path.restype = i32
    lib.ssd_chunk_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, shp, i32, vp, sz, vp]
    lib.ssd_chunk_scan_fwd.restype = i32
    lib.ssd_chunk_scan_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, shp, i32, vp, sz, vp,
                                          i32, ctypes.POINTER(vp), i32, ctypes.POINTER(i32),
                                          ctypes.POINTER(ctypes.c_char_p)]
    lib.ssd_chunk_scan_fwd_ex.restype = i32
    lib.ssd_chunk_scan_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, shp, i32, vp]
    lib.ssd_chunk_scan_fwd_noalloc.restype = i32
    lib.ssd_state_correction.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, shp, i32, vp]
    lib.ssd_state_correction.restype = i32
    lib.ssd_status_string.argtypes = [i32]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_last_error.argtypes = []
    lib.ssd_last_error.restype = ctypes.c_char_p
    lib.ssd_abi_version.argtypes = []
    lib.ssd_abi_version.restype = i32
    _lib = lib
    return lib


def ssd_abi_version() -> int:
    return int(_load().ssd_abi_version())


def ssd_status_string(status: int) -> str:
    return _load().ssd_status_string(status).decode()


def ssd_last_error() -> str:
    return _load().ssd_last_error().decode()


def _check(status: int):
    if status != 0:
        raise SsdError(status, ssd_last_error())


def make_shape(batch, seqlen, nheads, headdim, dstate, ngroups) -> ssd_shape:
    return ssd_shape(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate), int(ngroups))


def ssd_workspace_bytes(shape: ssd_shape, chunk_size: int, dtype: int) -> int:
    return int(_load().ssd_workspace_bytes(ctypes.byref(shape), int(chunk_size), int(dtype)))


def ssd_get_workspace_layout(shape: ssd_shape, chunk_size: int, dtype: int) -> ssd_workspace_layout:
    out = ssd_workspace_layout()
    _check(_load().ssd_get_workspace_layout(ctypes.byref(shape), int(chunk_size), int(dtype), ctypes.byref(out)))
    return out


def ssd_select_path(shape: ssd_shape, chunk_size: int, dtype: int) -> int:
    path = int(_load().ssd_select_path(ctypes.byref(shape), int(chunk_size), int(dtype)))
    if path < 0:
        raise SsdError(7, ssd_last_error())
    return path


def _dtype_code(torch, t) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_DTYPE_BF16
    if t.dtype == torch.float32:
        return SSD_DTYPE_F32
    raise TypeError(f"x must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def ssd_chunk_scan_fwd(x, dt, A, B, C, D=None, init_state=None, chunk_size: int = 256, state_out_idx=None, *,
                       y=None, final_state=None, return_final_state: bool = True, state_out=None,
                       workspace=None, stream=None):
    """Run the SSD forward on torch device tensors.

    x [b,T,H,P] bf16|fp32, dt [b,T,H] fp32, A [H] fp32, B/C [b,T,G,N] like x,
    D [H] fp32 or None, init_state [b,H,P,N] fp32 or None, state_out_idx [b]
    int32 or None.  Outputs are allocated when not given; given ones must
    have the exact shape, dtype and device.  Returns (y, final_state or None,
    state_out or None).  Raises ValueError/TypeError for a tensor that does
    not fit the call (before anything runs) and SsdError on any status other
    than SSD_OK.
    """
    y, final_state, state_out, _ = _run(x, dt, A, B, C, D, init_state, chunk_size, state_out_idx, y, final_state,
                                        return_final_state, state_out, workspace, stream, SSD_PATH_AUTO, None)
    return y, final_state, state_out


def ssd_chunk_scan_fwd_ex(x, dt, A, B, C, D=None, init_state=None, chunk_size: int = 256, state_out_idx=None, *,
                          path: int = SSD_PATH_AUTO, marks=(), y=None, final_state=None,
                          return_final_state: bool = True, state_out=None, workspace=None, stream=None):
    """ssd_chunk_scan_fwd on a chosen path (SSD_PATH_*), recording the HIP
    events `marks` (raw hipEvent_t handles as ints): marks[0] before the
    first kernel, marks[k] after the k-th.  Returns (y, final_state,
    state_out, names of the kernels that marks[1:] end)."""
    return _run(x, dt, A, B, C, D, init_state, chunk_size, state_out_idx, y, final_state, return_final_state,
                state_out, workspace, stream, int(path), list(marks))


def ssd_chunk_scan_fwd_noalloc(x, dt, A, B, C, D=None, init_state=None, chunk_size: int = 256,
                               state_out_idx=None, *, y=None, final_state=None, return_final_state: bool = True,
                               state_out=None, stream=None):
    """ssd_chunk_scan_fwd through the entry point that allocates nothing: a
    workspace, when the call needs one, is the library's static device
    scratch (at most SSD_NOALLOC_SCRATCH_BYTES).  Pass y, final_state and
    state_out to allocate nothing here either; missing ones are allocated
    by torch before the call."""
    y, final_state, state_out, _ = _run(x, dt, A, B, C, D, init_state, chunk_size, state_out_idx, y, final_state,
                                        return_final_state, state_out, None, stream, SSD_PATH_AUTO, None,
                                        noalloc=True)
    return y, final_state, state_out


def ssd_state_correction(y, dt, A, C, h_in, shard_final=None, final_state=None, state_out_idx=None,
                         state_out=None, *, stream=None):
    """Sequence-shard correction in place (see ssd_state_correction in
    include/ssd.h): y [b,T,H,P] holds the shard's outputs from a zero initial
    state and becomes those from h_in [b,H,P,N]; final_state (may be
    shard_final itself) receives shard_final + exp(cs_{T-1}) h_in; state_out,
    given with state_out_idx, gains exp(cs_j) h_in.  dt, A, C as for the
    shard's forward.  Returns (y, final_state, state_out)."""
    import torch

    if y.dim() != 4 or C.dim() != 4:
        raise ValueError("y must be [b,T,H,P] and C [b,T,G,N]")
    b, T, H, P = y.shape
    G, N = C.shape[2], C.shape[3]
    code = _dtype_code(torch, y)
    dev = y.device
    state_shape = (b, H, P, N)
    _expect("y", y, y.shape, y.dtype, dev)
    _expect("C", C, (b, T, G, N), y.dtype, dev)
    _expect("dt", dt, (b, T, H), torch.float32, dev)
    _expect("A", A, (H,), torch.float32, dev)
    _expect("h_in", h_in, state_shape, torch.float32, dev)
    if shard_final is not None:
        _expect("shard_final", shard_final, state_shape, torch.float32, dev)
    if final_state is not None:
        _expect("final_state", final_state, state_shape, torch.float32, dev)
    if state_out_idx is not None:
        _expect("state_out_idx", state_out_idx, (b,), torch.int32, dev)
    if state_out is not None:
        _expect("state_out", state_out, state_shape, torch.float32, dev)
    if (state_out is None) != (state_out_idx is None):
        raise ValueError("state_out and state_out_idx go together")
    if not y.is_cuda:
        raise ValueError(f"tensors must be on a GPU device, y is on {dev}")
    lib = _load()
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    _check(lib.ssd_state_correction(_ptr(y), _ptr(dt), _ptr(A), _ptr(C), _ptr(h_in), _ptr(shard_final),
                                    _ptr(final_state), _ptr(state_out_idx), _ptr(state_out),
                                    ctypes.byref(make_shape(b, T, H, P, N, G)), code,
                                    ctypes.c_void_p(stream) if stream else None))
    return y, final_state, state_out


def _expect(name, t, shape, dtype, device):
    """Checks one tensor argument; `shape` is the exact shape required."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, x on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _run(x, dt, A, B, C, D, init_state, chunk_size, state_out_idx, y, final_state, return_final_state, state_out,
         workspace, stream, path, marks, noalloc=False):
    import torch

    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b,T,H,P] and B, C [b,T,G,N]")
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(torch, x)
    dev = x.device
    state_shape = (b, H, P, N)
    _expect("x", x, x.shape, x.dtype, dev)
    _expect("B", B, (b, T, G, N), x.dtype, dev)
    _expect("C", C, (b, T, G, N), x.dtype, dev)
    _expect("dt", dt, (b, T, H), torch.float32, dev)
    _expect("A", A, (H,), torch.float32, dev)
    if D is not None:
        _expect("D", D, (H,), torch.float32, dev)
    if init_state is not None:
        _expect("init_state", init_state, state_shape, torch.float32, dev)
    if state_out_idx is not None:
        _expect("state_out_idx", state_out_idx, (b,), torch.int32, dev)
    elif state_out is not None:
        raise ValueError("state_out needs state_out_idx")
    if y is not None:
        _expect("y", y, x.shape, x.dtype, dev)
    if final_state is not None:
        _expect("final_state", final_state, state_shape, torch.float32, dev)
    if state_out is not None:
        _expect("state_out", state_out, state_shape, torch.float32, dev)
    if workspace is not None:
        if workspace.dim() != 1:
            raise ValueError("workspace must be a 1-D uint8 tensor")
        _expect("workspace", workspace, workspace.shape, torch.uint8, dev)
    if not x.is_cuda:
        raise ValueError(f"tensors must be on a GPU device, x is on {dev}")

    lib = _load()
    shape = make_shape(b, T, H, P, N, G)
    layout = ssd_get_workspace_layout(shape, chunk_size, code)  # raises the status of an invalid shape
    chosen = ssd_select_path(shape, chunk_size, code)
    run_path = path if path != SSD_PATH_AUTO and chosen != SSD_PATH_AUTO else chosen
    ws_bytes = layout.total_bytes if run_path == SSD_PATH_CHUNK_PARALLEL else 0
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty(state_shape, dtype=torch.float32, device=dev)
    if state_out_idx is not None and state_out is None:
        state_out = torch.empty(state_shape, dtype=torch.float32, device=dev)
    if workspace is None and ws_bytes > 0 and not noalloc:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    if noalloc:
        _check(lib.ssd_chunk_scan_fwd_noalloc(
            _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), int(chunk_size), _ptr(y),
            _ptr(final_state), _ptr(state_out_idx), _ptr(state_out), ctypes.byref(shape), code,
            ctypes.c_void_p(stream) if stream else None))
        return y, final_state, state_out, None
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), int(chunk_size), _ptr(y),
            _ptr(final_state), _ptr(state_out_idx), _ptr(state_out), ctypes.byref(shape), code, _ptr(workspace),
            int(workspace.numel()) if workspace is not None else 0, ctypes.c_void_p(stream) if stream else None)
    if marks is None:
        _check(lib.ssd_chunk_scan_fwd(*args))
        return y, final_state, state_out, None
    n = len(marks)
    arr = (ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(int(m)) for m in marks])
    names = (ctypes.c_char_p * max(n, 1))()
    count = ctypes.c_int(0)
    _check(lib.ssd_chunk_scan_fwd_ex(*args, int(path), arr, n, ctypes.byref(count), names))
    used = min(count.value, n - 1) if n > 0 else 0
    return y, final_state, state_out, [names[k].decode() for k in range(used)]


def workspace_views(workspace, shape: ssd_shape, chunk_size: int, dtype: int):
    """Views into the chunk-parallel path's workspace after a call, by the
    layout of include/ssd.h: cs, ct and dte [b,H,nc,Q] fp32, the chunk states
    from a zero start and the states entering each chunk (entry 0 only with
    init_state), both [b,nc,H,P,N] in the input dtype."""
    import torch

    lay = ssd_get_workspace_layout(shape, chunk_size, dtype)
    nc = lay.nchunks
    b, H, P, N = shape.batch, shape.nheads, shape.headdim, shape.dstate
    n_cs = b * H * nc * chunk_size
    n_st = b * nc * H * P * N
    tdt, esz = (torch.bfloat16, 2) if dtype == SSD_DTYPE_BF16 else (torch.float32, 4)

    def region(off, nbytes, dt, dims):
        return workspace[off:off + nbytes].view(dt).view(*dims)

    tab = (b, H, nc, chunk_size)
    return dict(cs=region(lay.cumsum_offset, 4 * n_cs, torch.float32, tab),
                ct=region(lay.ct_offset, 4 * n_cs, torch.float32, tab),
                dte=region(lay.dt_decay_offset, 4 * n_cs, torch.float32, tab),
                states=region(lay.states_offset, esz * n_st, tdt, (b, nc, H, P, N)),
                prev=region(lay.prev_offset, esz * n_st, tdt, (b, nc, H, P, N)))
