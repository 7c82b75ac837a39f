"""ctypes binding of libssd (include/ssd.h) for torch tensors.

Argument marshalling only: every step of the scan and of the recurrent step
runs in the HIP kernels of libssd.so.  There is no fallback: if the library
is not built, loading it raises.

    out, final = ssd_scan_fwd(x, dt, dt_bias, A, B, C, D, init_state, chunk=256)
    y = ssd_step(state, x, dt, A, B, C, D)          # state updated in place
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import struct
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libssd.so")

SSD_F32, SSD_BF16 = 0, 1
SSD_ALGO_AUTO, SSD_ALGO_FUSED, SSD_ALGO_CHUNKED, SSD_ALGO_ROWS, SSD_ALGO_QUAD = 0, 1, 2, 3, 4
STATUS = {0: "SSD_OK", 1: "SSD_ERR_NULL", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE",
          4: "SSD_ERR_LAYOUT", 5: "SSD_ERR_UNSUPPORTED", 6: "SSD_ERR_ALIAS",
          7: "SSD_ERR_NOMEM", 8: "SSD_ERR_HIP"}


class SsdTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("strides", ctypes.c_int64 * 4)]


class SsdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


_lib = None


def lib():
    """Load libssd.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libssd.so is not built (python -m mamba_ssd_scan_05_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        # tensor descriptors go in as addresses (ctypes pointers from
        # describe() are accepted too)
        P = ctypes.c_void_p
        L.ssd_scan_fwd.argtypes = [P] * 10 + [ctypes.c_int, ctypes.c_void_p]
        L.ssd_scan_fwd.restype = ctypes.c_int
        L.ssd_scan_fwd_algo.argtypes = [P] * 10 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.ssd_scan_fwd_algo.restype = ctypes.c_int
        L.ssd_scan_fwd_rows.argtypes = [P] * 10 + [ctypes.c_int, ctypes.c_void_p]
        L.ssd_scan_fwd_rows.restype = ctypes.c_int
        L.ssd_scan_fwd_gated.argtypes = [P] * 11 + [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.ssd_scan_fwd_gated.restype = ctypes.c_int
        L.ssd_selective_scan_fwd.argtypes = [P] * 10 + [ctypes.c_int, ctypes.c_void_p]
        L.ssd_selective_scan_fwd.restype = ctypes.c_int
        L.ssd_step.argtypes = [P] * 8 + [ctypes.c_void_p]
        L.ssd_scan_bwd.argtypes = [P] * 18 + [ctypes.c_void_p]
        L.ssd_scan_bwd.restype = ctypes.c_int
        L.ssd_scan_bwd_gated.argtypes = [P] * 20 + [ctypes.c_void_p]
        L.ssd_scan_bwd_gated.restype = ctypes.c_int
        L.ssd_step.restype = ctypes.c_int
        L.ssd_status_string.argtypes = [ctypes.c_int]
        L.ssd_status_string.restype = ctypes.c_char_p
        L.ssd_last_error.restype = ctypes.c_char_p
        L.ssd_version.restype = ctypes.c_int
        L.ssd_release_scratch.restype = ctypes.c_int
        L.ssd_release_scratch.argtypes = []
        L.ssd_scratch_stats.argtypes = [ctypes.POINTER(ctypes.c_int64)] * 2
        L.ssd_scratch_stats.restype = ctypes.c_int
        L.ssd_scan_fwd_noalloc.argtypes = [P] * 10 + [ctypes.c_int, ctypes.c_void_p]
        L.ssd_scan_fwd_noalloc.restype = ctypes.c_int
        L.ssd_fixed_scratch_bytes.argtypes = []
        L.ssd_fixed_scratch_bytes.restype = ctypes.c_int64
        L.ssd_scan_plan.argtypes = [ctypes.c_int64] * 6 + [ctypes.c_int, ctypes.c_int,
                                                            ctypes.POINTER(ctypes.c_int),
                                                            ctypes.POINTER(ctypes.c_int)]
        L.ssd_scan_plan.restype = ctypes.c_int
        _lib = L
    return _lib


_DTYPE_CODE = {torch.float32: SSD_F32, torch.bfloat16: SSD_BF16}


def _dtype_code(t: torch.Tensor) -> int:
    return _DTYPE_CODE.get(t.dtype, 99)  # 99: rejected by the library as SSD_ERR_DTYPE


def describe(t: Optional[torch.Tensor]):
    """ssd_tensor descriptor of a torch tensor (None -> NULL pointer)."""
    if t is None:
        return None
    if t.dim() > 4:
        raise ValueError("ssd tensors have at most 4 dimensions")
    d = SsdTensor()
    d.data = t.data_ptr() if t.numel() else 0
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i, (s, st) in enumerate(zip(t.shape, t.stride())):
        d.shape[i] = s
        d.strides[i] = st
    return ctypes.pointer(d)


# ssd_tensor as packed bytes: data, dtype, ndim, shape[4], strides[4]
_DESC = struct.Struct("<Qii4q4q")
assert _DESC.size == ctypes.sizeof(SsdTensor)


def _descs(*ts):
    """Descriptors of a call's tensors in one buffer: (buffer, addresses),
    None -> NULL.  Keep the buffer alive until the call returns."""
    buf = ctypes.create_string_buffer(_DESC.size * len(ts))
    base = ctypes.addressof(buf)
    addrs = []
    for i, t in enumerate(ts):
        if t is None:
            addrs.append(None)
            continue
        n = t.dim()
        if n > 4:
            raise ValueError("ssd tensors have at most 4 dimensions")
        pad = (0,) * (4 - n)
        _DESC.pack_into(buf, i * _DESC.size, t.data_ptr() if t.numel() else 0, _dtype_code(t), n,
                        *t.shape, *pad, *t.stride(), *pad)
        addrs.append(base + i * _DESC.size)
    return buf, addrs


def _on_device(t):
    """Make t's device current for the call (the library launches on the
    current device and refuses memory that device cannot address)."""
    if t is not None and t.is_cuda and t.device.index != torch.cuda.current_device():
        return torch.cuda.device(t.device)
    return contextlib.nullcontext()


def _stream(stream, t):
    if stream is not None:
        return stream
    if t is not None and t.is_cuda:
        return torch.cuda.current_stream(t.device).cuda_stream
    return None


def _check(status: int):
    if status != 0:
        raise SsdError(status, lib().ssd_last_error().decode())


def ssd_scan_fwd(x, dt, dt_bias, A, B, C, D=None, init_state=None, out=None,
                 final_state=None, chunk: int = 256, stream=None,
                 algo: int = SSD_ALGO_AUTO, return_final_state: bool = True):
    """Forward SSD scan; returns (out, final_state or None)."""
    if out is None:
        out = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty((x.shape[0], x.shape[2], x.shape[3], B.shape[3]),
                                  dtype=torch.float32, device=x.device)
    keep, d = _descs(x, dt, dt_bias, A, B, C, D, init_state, out, final_state)
    with _on_device(x):
        st = _stream(stream, x)
        if algo == SSD_ALGO_AUTO:
            # the library's own plan: the plain entry point
            status = lib().ssd_scan_fwd(*d, int(chunk), st)
        else:
            status = lib().ssd_scan_fwd_algo(*d, int(chunk), int(algo), st)
    _check(status)
    return out, final_state


def ssd_scan_fwd_noalloc(x, dt, dt_bias, A, B, C, D=None, init_state=None, out=None,
                         final_state=None, chunk: int = 256, stream=None):
    """ssd_scan_fwd through the allocation-free entry point (scratch in the
    library's fixed device array).  out (and final_state, if wanted) should
    be passed in by callers that cannot allocate; returns (out, final_state)."""
    if out is None:
        out = torch.empty_like(x)
    with _on_device(x):
        st = _stream(stream, x)
        keep, d = _descs(x, dt, dt_bias, A, B, C, D, init_state, out, final_state)
        status = lib().ssd_scan_fwd_noalloc(*d, int(chunk), st)
    _check(status)
    return out, final_state


def ssd_fixed_scratch_bytes() -> int:
    return int(lib().ssd_fixed_scratch_bytes())


def ssd_scratch_stats():
    """(number of kept scratch buffers, their total bytes)."""
    n, t = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().ssd_scratch_stats(ctypes.byref(n), ctypes.byref(t)))
    return n.value, t.value


def ssd_scan_bwd(x, dt, dt_bias, A, B, C, D, init_state, dout, dfinal_state=None, *,
                 want_dt_bias: bool = True, want_D: bool = True, want_init: bool = True,
                 out: dict = None, stream=None):
    """Gradients of ssd_scan_fwd for the objective <dout, y> + <dfinal_state, final state>.

    Returns a dict of fp32 tensors: dx, ddt (at the raw dt), dA, dB, dC and,
    when asked for, ddt_bias, dD, dinit.  ``out`` may hold preallocated
    tensors under those names."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    shapes = dict(dx=(b, L, H, P), ddt=(b, L, H), dA=(H,), dB=(b, L, G, N), dC=(b, L, G, N),
                  ddt_bias=(H,) if want_dt_bias else None, dD=(H,) if want_D else None,
                  dinit=(b, H, P, N) if want_init else None)
    g = dict(out or {})
    for k, shp in shapes.items():
        if shp is not None and g.get(k) is None:
            g[k] = torch.empty(shp, dtype=torch.float32, device=dev)
        elif shp is None:
            g[k] = None
    with _on_device(x):
        st = _stream(stream, x)
        keep, d = _descs(x, dt, dt_bias, A, B, C, D, init_state, dout, dfinal_state,
                         g["dx"], g["ddt"], g["ddt_bias"], g["dA"], g["dB"], g["dC"], g["dD"], g["dinit"])
        status = lib().ssd_scan_bwd(*d, st)
    _check(status)
    return g


def ssd_scan_bwd_gated(x, dt, dt_bias, A, B, C, z, D, init_state, dout, dfinal_state=None, *,
                       want_dt_bias: bool = True, want_D: bool = True, want_init: bool = True,
                       out: dict = None, stream=None):
    """Gradients of ssd_scan_fwd_gated (out = y * silu(z)); the dict of
    ssd_scan_bwd plus dz (fp32)."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    dev = x.device
    shapes = dict(dx=(b, L, H, P), ddt=(b, L, H), dA=(H,), dB=(b, L, G, N), dC=(b, L, G, N),
                  ddt_bias=(H,) if want_dt_bias else None, dD=(H,) if want_D else None,
                  dinit=(b, H, P, N) if want_init else None, dz=(b, L, H, P))
    g = dict(out or {})
    for k, shp in shapes.items():
        if shp is not None and g.get(k) is None:
            g[k] = torch.empty(shp, dtype=torch.float32, device=dev)
        elif shp is None:
            g[k] = None
    with _on_device(x):
        st = _stream(stream, x)
        keep, d = _descs(x, dt, dt_bias, A, B, C, D, z, init_state, dout, dfinal_state,
                         g["dx"], g["ddt"], g["ddt_bias"], g["dA"], g["dB"], g["dC"], g["dD"], g["dz"],
                         g["dinit"])
        status = lib().ssd_scan_bwd_gated(*d, st)
    _check(status)
    return g


def ssd_scan_fwd_gated(x, dt, dt_bias, A, B, C, z, D=None, init_state=None, out=None,
                       final_state=None, chunk: int = 256, stream=None,
                       algo: int = SSD_ALGO_AUTO, return_final_state: bool = True):
    """Forward scan with the output gate: out = y * silu(z); returns
    (out, final_state or None)."""
    if out is None:
        out = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty((x.shape[0], x.shape[2], x.shape[3], B.shape[3]),
                                  dtype=torch.float32, device=x.device)
    with _on_device(x):
        st = _stream(stream, x)
        keep, d = _descs(x, dt, dt_bias, A, B, C, D, z, init_state, out, final_state)
        status = lib().ssd_scan_fwd_gated(*d, int(chunk), int(algo), st)
    _check(status)
    return out, final_state


def ssd_scan_fwd_rows(x, dt, dt_bias, A, B, C, D=None, init_state=None, out=None,
                      final_state=None, waves: int = 0, stream=None,
                      return_final_state: bool = True):
    """Row-sliced walk with `waves` waves per workgroup (0 = automatic)."""
    if out is None:
        out = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty((x.shape[0], x.shape[2], x.shape[3], B.shape[3]),
                                  dtype=torch.float32, device=x.device)
    with _on_device(x):
        st = _stream(stream, x)
        keep, d = _descs(x, dt, dt_bias, A, B, C, D, init_state, out, final_state)
        status = lib().ssd_scan_fwd_rows(*d, int(waves), st)
    _check(status)
    return out, final_state


def ssd_selective_scan_fwd(x, dt, dt_bias, A, B, C, D=None, init_state=None, out=None,
                           final_state=None, segments: int = 0, stream=None,
                           return_final_state: bool = True):
    """Selective scan with a diagonal A [D, N] per (channel, state index);
    x, dt [b, L, D]; returns (out, final_state or None)."""
    if out is None:
        out = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty((x.shape[0], x.shape[2], B.shape[3]), dtype=torch.float32,
                                  device=x.device)
    with _on_device(x):
        st = _stream(stream, x)
        keep, d = _descs(x, dt, dt_bias, A, B, C, D, init_state, out, final_state)
        status = lib().ssd_selective_scan_fwd(*d, int(segments), st)
    _check(status)
    return out, final_state


def ssd_step(state, x, dt, A, B, C, D=None, out=None, stream=None):
    """One recurrent step; ``state`` is updated in place; returns out."""
    if out is None:
        out = torch.empty_like(x)
    with _on_device(state):
        st = _stream(stream, state)
        keep, d = _descs(state, x, dt, A, B, C, D, out)
        status = lib().ssd_step(*d, st)
    _check(status)
    return out


def ssd_scan_plan(b, L, H, P, G, N, dtype=torch.bfloat16, cus: int = 256):
    """(algo, seg_len) that SSD_ALGO_AUTO uses for this shape and input dtype."""
    algo, seg = ctypes.c_int(), ctypes.c_int()
    code = SSD_BF16 if dtype in (torch.bfloat16, SSD_BF16) else SSD_F32
    _check(lib().ssd_scan_plan(b, L, H, P, G, N, code, cus, ctypes.byref(algo), ctypes.byref(seg)))
    return algo.value, seg.value


def ssd_status_string(status: int) -> str:
    return lib().ssd_status_string(int(status)).decode()


def ssd_last_error() -> str:
    return lib().ssd_last_error().decode()


def ssd_version() -> int:
    return int(lib().ssd_version())


def ssd_release_scratch() -> None:
    """Frees the scratch buffers the library keeps between calls (waits for
    the queued work that uses them)."""
    _check(lib().ssd_release_scratch())
