"""fp64 CPU oracle for the Mamba-2 SSD scan (test infrastructure).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers.  The HIP library and its
Python binding never import this package, and this package imports nothing
from them.

The arithmetic lives in ``ssd_oracle.c`` (plain sequential recurrence in
float64, see that file for the page citations).  This module only builds it
with gcc, loads it with ctypes and marshals numpy arrays:

* ``scan(x, dt, dt_bias, A, B, C, D, init)`` -> ``(y, final_state)``
* ``scan_gated(x, dt, dt_bias, A, B, C, z, D, init)`` -> ``(y * silu(z), final_state)``
* ``gate(y, z)`` -> ``y * silu(z)``
* ``step(state, x, delta, A, B, C, D)`` -> ``(y, new_state)``
* ``scan_bwd(x, dt, dt_bias, A, B, C, D, init, dy, dfinal)`` -> dict of gradients
* ``scan_bwd_gated(x, dt, dt_bias, A, B, C, z, D, init, dout, dfinal)`` -> the same plus dz

Every array argument is converted to contiguous float64 first; callers pass
the values exactly as the device sees them (bf16 inputs upcast exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libssd_oracle.so")
_default = None


def compile_source(src: str, out: str) -> str:
    """Compile one oracle C source into a shared library with gcc + OpenMP."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-Wall", "-Werror", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ssd_oracle.c into libssd_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


class Oracle:
    """ctypes front end of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_scan_f64.argtypes = [i64] * 6 + [vp] * 10
        lib.oracle_scan_f64.restype = None
        lib.oracle_step_f64.argtypes = [i64] * 5 + [vp] * 8
        lib.oracle_step_f64.restype = None
        lib.oracle_gate_f64.argtypes = [i64, vp, vp, vp]
        lib.oracle_gate_f64.restype = None
        lib.oracle_sscan_f64.argtypes = [i64] * 5 + [vp] * 10
        lib.oracle_sscan_f64.restype = None
        lib.oracle_scan_bwd_f64.argtypes = [i64] * 6 + [vp] * 18
        lib.oracle_scan_bwd_f64.restype = None
        lib.oracle_gate_bwd_f64.argtypes = [i64] + [vp] * 5
        lib.oracle_gate_bwd_f64.restype = None
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        self.lib = lib

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def scan(self, *args, **kwargs):
        return _scan(self.lib, *args, **kwargs)

    def step(self, *args, **kwargs):
        return _step(self.lib, *args, **kwargs)

    def gate(self, y, z):
        return _gate(self.lib, y, z)

    def selective_scan(self, *args, **kwargs):
        return _sscan(self.lib, *args, **kwargs)

    def scan_bwd(self, *args, **kwargs):
        return _scan_bwd(self.lib, *args, **kwargs)

    def scan_bwd_gated(self, *args, **kwargs):
        return _scan_bwd_gated(self, *args, **kwargs)


def default() -> Oracle:
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        _default = Oracle(_LIB_PATH)
    return _default


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan_bwd(x, dt, dt_bias, A, B, C, D, init, dy, dfinal=None):
    return default().scan_bwd(x, dt, dt_bias, A, B, C, D, init, dy, dfinal)


def scan_bwd_gated(x, dt, dt_bias, A, B, C, z, D, init, dout, dfinal=None):
    return default().scan_bwd_gated(x, dt, dt_bias, A, B, C, z, D, init, dout, dfinal)


def scan(x, dt, dt_bias, A, B, C, D=None, init=None, want_final=True):
    """Sequential fp64 scan (see ``_scan``)."""
    return default().scan(x, dt, dt_bias, A, B, C, D, init, want_final)


def step(state, x, delta, A, B, C, D=None):
    """One fp64 recurrent step (see ``_step``)."""
    return default().step(state, x, delta, A, B, C, D)


def gate(y, z):
    """Elementwise y * silu(z) in fp64 (see ``_gate``)."""
    return default().gate(y, z)


def selective_scan(x, dt, dt_bias, A, B, C, D=None, init=None, want_final=True):
    """Sequential fp64 selective scan with a diagonal A per (channel, n)
    (see ``_sscan``)."""
    return default().selective_scan(x, dt, dt_bias, A, B, C, D, init, want_final)


def scan_gated(x, dt, dt_bias, A, B, C, z, D=None, init=None, want_final=True):
    """The scan followed by the output gate: (y * silu(z), final_state)."""
    y, fin = scan(x, dt, dt_bias, A, B, C, D, init, want_final)
    return gate(y, z), fin


def _scan(lib, x, dt, dt_bias, A, B, C, D=None, init=None, want_final=True):
    """Sequential fp64 scan.

    x [b,L,H,P], dt [b,L,H] (raw, before softplus), dt_bias [H] or None,
    A [H], B/C [b,L,G,N], D [H] or None, init [b,H,P,N] or None.
    Returns (y [b,L,H,P], final_state [b,H,P,N] or None), float64.
    """
    x, dt, dt_bias, A, B, C, D, init = map(_f64, (x, dt, dt_bias, A, B, C, D, init))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, L, H) and A.shape == (H,)
    assert B.shape == (b, L, G, N) and C.shape == (b, L, G, N)
    assert H % G == 0
    if dt_bias is not None:
        assert dt_bias.shape == (H,)
    if D is not None:
        assert D.shape == (H,)
    if init is not None:
        assert init.shape == (b, H, P, N)
    y = np.empty((b, L, H, P), np.float64)
    fin = np.empty((b, H, P, N), np.float64) if want_final else None
    lib.oracle_scan_f64(b, L, H, P, G, N, _ptr(x), _ptr(dt), _ptr(dt_bias),
                        _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(init),
                        _ptr(y), _ptr(fin))
    return y, fin


def _step(lib, state, x, delta, A, B, C, D=None):
    """One fp64 recurrent step on a copy of ``state``.

    state [b,H,P,N], x [b,H,P], delta [b,H] (already activated),
    A [H], B/C [b,G,N], D [H] or None.  Returns (y [b,H,P], new_state).
    """
    S = np.array(state, dtype=np.float64, order="C", copy=True)
    x, delta, A, B, C, D = map(_f64, (x, delta, A, B, C, D))
    b, H, P, N = S.shape
    G = B.shape[1]
    assert x.shape == (b, H, P) and delta.shape == (b, H)
    assert B.shape == (b, G, N) and C.shape == (b, G, N) and H % G == 0
    y = np.empty((b, H, P), np.float64)
    lib.oracle_step_f64(b, H, P, G, N, _ptr(S), _ptr(x), _ptr(delta),
                        _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(y))
    return y, S


def _gate(lib, y, z):
    """out = y * silu(z), silu(v) = v / (1 + e^-v), elementwise, float64."""
    y, z = _f64(y), _f64(z)
    assert y.shape == z.shape
    out = np.empty_like(y)
    lib.oracle_gate_f64(y.size, _ptr(y), _ptr(z), _ptr(out))
    return out


def _sscan(lib, x, dt, dt_bias, A, B, C, D=None, init=None, want_final=True):
    """Sequential fp64 selective scan, diagonal A per (channel, state index).

    x, dt [b,L,Dc] (dt raw, before softplus), dt_bias [Dc] or None,
    A [Dc,N], B/C [b,L,G,N] (channel d reads group floor(d*G/Dc)),
    D [Dc] or None, init [b,Dc,N] or None.  Returns (y [b,L,Dc],
    final_state [b,Dc,N] or None) in float64.  Follows oracle_sscan_f64 in
    ssd_oracle.c (Mamba paper-reading notes, selective mechanism)."""
    x, dt, A, B, C = (_f64(v) for v in (x, dt, A, B, C))
    dt_bias, D, init = _f64(dt_bias), _f64(D), _f64(init)
    b, L, Dc = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, L, Dc) and A.shape == (Dc, N)
    assert B.shape == (b, L, G, N) and C.shape == B.shape
    y = np.empty((b, L, Dc), dtype=np.float64)
    fin = np.empty((b, Dc, N), dtype=np.float64) if want_final else None
    lib.oracle_sscan_f64(b, L, Dc, G, N, _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B),
                         _ptr(C), _ptr(D), _ptr(init), _ptr(y), _ptr(fin))
    return y, fin


def _scan_bwd(lib, x, dt, dt_bias, A, B, C, D, init, dy, dfinal=None):
    """Gradients of the sequential fp64 scan (oracle_scan_bwd_f64 in
    ssd_oracle.c: the chain rule through the recurrence, latest token first).

    Arguments as for ``scan`` plus dy [b,L,H,P] (gradient at y) and dfinal
    [b,H,P,N] or None (gradient at the final state).  Returns a dict of
    float64 arrays: dx [b,L,H,P], ddt [b,L,H] (at the raw dt), ddt_bias,
    dA and dD [H], dB and dC [b,L,G,N], dinit [b,H,P,N]."""
    x, dt, dt_bias, A, B, C, D, init, dy, dfinal = map(
        _f64, (x, dt, dt_bias, A, B, C, D, init, dy, dfinal))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (b, L, H) and A.shape == (H,) and H % G == 0
    assert B.shape == (b, L, G, N) and C.shape == (b, L, G, N) and dy.shape == x.shape
    if dfinal is not None:
        assert dfinal.shape == (b, H, P, N)
    out = dict(dx=np.empty((b, L, H, P)), ddt=np.empty((b, L, H)), ddt_bias=np.empty(H),
               dA=np.empty(H), dB=np.empty((b, L, G, N)), dC=np.empty((b, L, G, N)),
               dD=np.empty(H), dinit=np.empty((b, H, P, N)))
    lib.oracle_scan_bwd_f64(b, L, H, P, G, N, _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B),
                            _ptr(C), _ptr(D), _ptr(init), _ptr(dy), _ptr(dfinal),
                            _ptr(out["dx"]), _ptr(out["ddt"]), _ptr(out["ddt_bias"]), _ptr(out["dA"]),
                            _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["dinit"]))
    return out


def _scan_bwd_gated(o, x, dt, dt_bias, A, B, C, z, D, init, dout, dfinal=None):
    """Gradients of the gated scan out = y * silu(z) (y the scan output with
    the D term): the scan's own y, then the gate's derivative
    (oracle_gate_bwd_f64: dy = dout * silu(z), dz = dout * y * silu'(z)), then
    the scan's gradients for dy.  Returns scan_bwd's dict plus dz."""
    y, _ = o.scan(x, dt, dt_bias, A, B, C, D, init, want_final=False)
    z, dout = _f64(z), _f64(dout)
    assert z.shape == y.shape and dout.shape == y.shape
    dy = np.empty_like(y)
    dz = np.empty_like(y)
    o.lib.oracle_gate_bwd_f64(y.size, _ptr(y), _ptr(z), _ptr(dout), _ptr(dy), _ptr(dz))
    g = o.scan_bwd(x, dt, dt_bias, A, B, C, D, init, dy, dfinal)
    g["dz"] = dz
    return g
