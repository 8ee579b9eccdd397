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
    "ssd_get_workspace_layout", "ssd_chunk_scan_fwd", "ssd_chunk_scan_fwd_marked", "workspace_views",
    "library_path",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libssd.so")
_lib = None

SSD_DTYPE_F32 = 0
SSD_DTYPE_BF16 = 1
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_CHUNK", 4: "SSD_ERR_ALIGN",
          5: "SSD_ERR_WORKSPACE", 6: "SSD_ERR_ALIAS", 7: "SSD_ERR_ARGS", 8: "SSD_ERR_HIP",
          9: "SSD_ERR_UNSUPPORTED"}


class ssd_shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64)]


class ssd_workspace_layout(ctypes.Structure):
    _fields_ = [("cumsum_offset", ctypes.c_size_t), ("ct_offset", ctypes.c_size_t),
                ("dt_decay_offset", ctypes.c_size_t), ("block_decay_offset", ctypes.c_size_t),
                ("states_offset", ctypes.c_size_t),
                ("prev_offset", ctypes.c_size_t), ("hj_offset", ctypes.c_size_t),
                ("sync_offset", ctypes.c_size_t), ("total_bytes", ctypes.c_size_t),
                ("nchunks", ctypes.c_int64)]


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
    lib.ssd_chunk_scan_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, shp, i32, vp, sz, vp]
    lib.ssd_chunk_scan_fwd.restype = i32
    lib.ssd_chunk_scan_fwd_marked.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, shp, i32, vp, sz, vp,
                                              ctypes.POINTER(vp), i32, ctypes.POINTER(i32),
                                              ctypes.POINTER(ctypes.c_char_p)]
    lib.ssd_chunk_scan_fwd_marked.restype = i32
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
    int32 or None.  Outputs are allocated when not given.  Returns
    (y, final_state or None, state_out or None).  Raises SsdError on any
    status other than SSD_OK.
    """
    y, final_state, state_out, _ = _run(x, dt, A, B, C, D, init_state, chunk_size, state_out_idx, y, final_state,
                                        return_final_state, state_out, workspace, stream, None)
    return y, final_state, state_out


def ssd_chunk_scan_fwd_marked(x, dt, A, B, C, D=None, init_state=None, chunk_size: int = 256,
                              state_out_idx=None, *, marks, y=None, final_state=None,
                              return_final_state: bool = True, state_out=None, workspace=None, stream=None):
    """ssd_chunk_scan_fwd that also records the HIP events `marks` (raw
    hipEvent_t handles as ints): marks[0] before the first kernel, marks[k]
    after the k-th.  Returns (y, final_state, state_out, kernel_names)."""
    return _run(x, dt, A, B, C, D, init_state, chunk_size, state_out_idx, y, final_state, return_final_state,
                state_out, workspace, stream, marks)


def _run(x, dt, A, B, C, D, init_state, chunk_size, state_out_idx, y, final_state, return_final_state, state_out,
         workspace, stream, marks):
    import torch

    lib = _load()
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [b,T,H,P] and B, C [b,T,G,N]")
    b, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    code = _dtype_code(torch, x)
    for name, t, dtype in (("dt", dt, torch.float32), ("A", A, torch.float32), ("B", B, x.dtype),
                           ("C", C, x.dtype), ("D", D, torch.float32), ("init_state", init_state, torch.float32),
                           ("state_out_idx", state_out_idx, torch.int32)):
        if t is None:
            continue
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if t.device != x.device:
            raise ValueError(f"{name} is on {t.device}, x on {x.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    shape = make_shape(b, T, H, P, N, G)
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    if state_out_idx is not None and state_out is None:
        state_out = torch.empty((b, H, P, N), dtype=torch.float32, device=x.device)
    ws_bytes = ssd_workspace_bytes(shape, chunk_size, code)
    if ws_bytes == 0 and b * T > 0:
        raise SsdError(2, ssd_last_error())
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    if stream is None:
        stream = torch.cuda.current_stream(x.device).cuda_stream if x.is_cuda else None
    args = (_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init_state), int(chunk_size), _ptr(y),
            _ptr(final_state), _ptr(state_out_idx), _ptr(state_out), ctypes.byref(shape), code, _ptr(workspace),
            int(workspace.numel()), ctypes.c_void_p(stream) if stream else None)
    if marks is None:
        _check(lib.ssd_chunk_scan_fwd(*args))
        return y, final_state, state_out, None
    n = len(marks)
    arr = (ctypes.c_void_p * max(n, 1))(*[ctypes.c_void_p(int(m)) for m in marks])
    names = (ctypes.c_char_p * max(n, 1))()
    count = ctypes.c_int(0)
    _check(lib.ssd_chunk_scan_fwd_marked(*args, arr, n, ctypes.byref(count), names))
    used = min(count.value, n - 1) if n > 0 else 0
    return y, final_state, state_out, [names[k].decode() for k in range(used)]


def workspace_views(workspace, shape: ssd_shape, chunk_size: int, dtype: int):
    """Views into a workspace after a call: cs [b,H,nc,Q] fp32, the chunk
    states from a zero start [b,nc,H,P,N] fp32, and the states entering each
    chunk [b,nc,H,P,N] in the input dtype (entry 0 only with init_state)."""
    import torch

    lay = ssd_get_workspace_layout(shape, chunk_size, dtype)
    nc = lay.nchunks
    b, H, P, N = shape.batch, shape.nheads, shape.headdim, shape.dstate
    n_cs = b * H * nc * chunk_size
    n_st = b * nc * H * P * N
    tdt, esz = (torch.bfloat16, 2) if dtype == SSD_DTYPE_BF16 else (torch.float32, 4)
    cs = workspace[lay.cumsum_offset:lay.cumsum_offset + 4 * n_cs].view(torch.float32).view(b, H, nc, chunk_size)
    st = workspace[lay.states_offset:lay.states_offset + 4 * n_st].view(torch.float32).view(b, nc, H, P, N)
    prev = workspace[lay.prev_offset:lay.prev_offset + esz * n_st].view(tdt).view(b, nc, H, P, N)
    return cs, st, prev
