"""Seeded synthetic inputs for the SSD scan and the recurrent step.

This module only draws random numbers and rounds them to the storage
dtypes; it performs none of the scan's arithmetic.  Both the HIP path (via
the tests and the benchmark) and the fp64 oracle consume exactly the arrays
produced here.

Distributions (the workload recipe, one per named workload):

* ``A_h = -exp(U(log 1, log 16))``                      per head, fp32
* ``dt_h = exp(U(log lo, log hi))``, ``dt_bias_h = softplus^-1(dt_h)``
  (``lo, hi = 1e-3, 0.1``; the long-sequence workload uses 1e-4, 1e-2)
* ``D_h ~ N(0, 1)``                                      fp32
* ``x ~ N(0, 1)``                                        bf16 or fp32
* ``dt_raw ~ 0.5 * N(0, 1)``                             fp32 (pre-activation)
* ``B, C ~ N(0, 1) / sqrt(N)``                           bf16 or fp32
* optional initial state ``~ N(0, std^2)``               fp32

Draw order is fixed (A, dt_h, D, x, dt_raw, B, C, init) from
``numpy.random.Generator(PCG64(seed))``.  Values are drawn in float64,
rounded to float32 (round-to-nearest-even), and bf16 tensors are further
rounded from float32 to bf16 with round-to-nearest-even; bf16 arrays are
returned as their uint16 bit patterns.

The recurrent step takes the activated step size as its input, so its
sampler draws ``dt_raw`` and applies the softplus to it here: that is the
step's input distribution, not a computation of the step.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

BF16 = "bf16"
F32 = "f32"


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest even); returns uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 view of a stored array (bf16 bits or float32)."""
    if dtype == BF16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _store(v64: np.ndarray, dtype: str) -> np.ndarray:
    v32 = v64.astype(np.float32)
    return f32_to_bf16_bits(v32) if dtype == BF16 else v32


def _inv_softplus(d: np.ndarray) -> np.ndarray:
    # softplus^-1(d) = log(e^d - 1) = d + log(-expm1(-d)), evaluated in fp64.
    return d + np.log(-np.expm1(-d))


def _softplus(z: np.ndarray) -> np.ndarray:
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


@dataclasses.dataclass
class ScanInputs:
    """Host arrays for one scan call.  bf16 tensors hold uint16 bits."""
    dtype: str
    chunk: int
    x: np.ndarray          # [b,L,H,P]
    dt: np.ndarray         # [b,L,H]  f32
    dt_bias: np.ndarray    # [H]      f32
    A: np.ndarray          # [H]      f32
    B: np.ndarray          # [b,L,G,N]
    C: np.ndarray          # [b,L,G,N]
    D: np.ndarray          # [H]      f32
    init: Optional[np.ndarray]  # [b,H,P,N] f32 or None

    @property
    def shape(self):
        b, L, H, P = self.x.shape
        return dict(b=b, L=L, H=H, P=P, G=self.B.shape[2], N=self.B.shape[3])

    def f64(self):
        """Exact float64 copies, in oracle argument order."""
        return dict(x=to_f64(self.x, self.dtype), dt=to_f64(self.dt, F32),
                    dt_bias=to_f64(self.dt_bias, F32), A=to_f64(self.A, F32),
                    B=to_f64(self.B, self.dtype), C=to_f64(self.C, self.dtype),
                    D=to_f64(self.D, F32),
                    init=None if self.init is None else to_f64(self.init, F32))


def make_scan(b, L, H, P, G, N, *, dtype=BF16, chunk=256, seed=0,
              dt_range=(1e-3, 0.1), init_std: Optional[float] = None,
              A_range=(1.0, 16.0)) -> ScanInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    A = -np.exp(rng.uniform(np.log(A_range[0]), np.log(A_range[1]), size=H))
    dt_h = np.exp(rng.uniform(np.log(dt_range[0]), np.log(dt_range[1]), size=H))
    D = rng.standard_normal(H)
    x = rng.standard_normal((b, L, H, P))
    dt_raw = 0.5 * rng.standard_normal((b, L, H))
    Bm = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    init = None
    if init_std is not None:
        init = init_std * rng.standard_normal((b, H, P, N))
    return ScanInputs(
        dtype=dtype, chunk=chunk,
        x=_store(x, dtype), dt=dt_raw.astype(np.float32),
        dt_bias=_inv_softplus(dt_h).astype(np.float32),
        A=A.astype(np.float32), B=_store(Bm, dtype), C=_store(Cm, dtype),
        D=D.astype(np.float32),
        init=None if init is None else init.astype(np.float32))


def make_gate(si: ScanInputs, seed: int = 100, scale: float = 1.5) -> np.ndarray:
    """Gate input z for a scan's output gate: the shape of x, drawn from
    N(0, scale^2) (so both tails of silu are used), stored in the scan's
    dtype (bf16 as uint16 bits)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _store(scale * rng.standard_normal(si.x.shape), si.dtype)


@dataclasses.dataclass
class StepInputs:
    """Host arrays for T consecutive recurrent steps (bf16 as uint16 bits)."""
    dtype: str
    state: np.ndarray      # [b,H,P,N] f32 (initial)
    x: np.ndarray          # [T,b,H,P]
    delta: np.ndarray      # [T,b,H]   f32, activated step sizes
    A: np.ndarray          # [H]
    B: np.ndarray          # [T,b,G,N]
    C: np.ndarray          # [T,b,G,N]
    D: np.ndarray          # [H]


def make_step(b, H, P, G, N, T, *, dtype=BF16, seed=4, dt_range=(1e-3, 0.1),
              state_std=1.0) -> StepInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    A = -np.exp(rng.uniform(0.0, np.log(16.0), size=H))
    dt_h = np.exp(rng.uniform(np.log(dt_range[0]), np.log(dt_range[1]), size=H))
    D = rng.standard_normal(H)
    x = rng.standard_normal((T, b, H, P))
    dt_raw = 0.5 * rng.standard_normal((T, b, H))
    Bm = rng.standard_normal((T, b, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((T, b, G, N)) / np.sqrt(N)
    state = state_std * rng.standard_normal((b, H, P, N))
    bias32 = _inv_softplus(dt_h).astype(np.float32).astype(np.float64)
    delta = _softplus(dt_raw.astype(np.float32).astype(np.float64) + bias32)
    return StepInputs(dtype=dtype, state=state.astype(np.float32),
                      x=_store(x, dtype), delta=delta.astype(np.float32),
                      A=A.astype(np.float32), B=_store(Bm, dtype),
                      C=_store(Cm, dtype), D=D.astype(np.float32))


# The five named workloads: four scans and one decode-step loop.
WORKLOADS = {
    "tiny_fp32_b1_L256_H4_P16_N16": dict(
        kind="scan", b=1, L=256, H=4, P=16, G=1, N=16, dtype=F32, chunk=64, seed=0),
    "mamba2_370m_b8_L2048_H32_P64_N128": dict(
        kind="scan", b=8, L=2048, H=32, P=64, G=1, N=128, dtype=BF16, chunk=256, seed=1),
    "mamba2_2p7b_b4_L4096_H80_P64_N128": dict(
        kind="scan", b=4, L=4096, H=80, P=64, G=1, N=128, dtype=BF16, chunk=256, seed=2,
        init_std=0.1),
    "long_gva_b1_L65536_H32_G8_P64_N128": dict(
        kind="scan", b=1, L=65536, H=32, P=64, G=8, N=128, dtype=BF16, chunk=256, seed=3,
        dt_range=(1e-4, 1e-2)),
    "decode_step_b256_H80_P64_N128_T64": dict(
        kind="step", b=256, H=80, P=64, G=1, N=128, T=64, dtype=BF16, seed=4),
}
WORKLOAD_ORDER = list(WORKLOADS)


@dataclasses.dataclass
class SScanInputs:
    """Host arrays for one selective scan with a diagonal A per (channel,
    state index).  bf16 tensors hold uint16 bits."""
    dtype: str
    x: np.ndarray          # [b,L,D]
    dt: np.ndarray         # [b,L,D]  f32 (raw)
    dt_bias: np.ndarray    # [D]      f32
    A: np.ndarray          # [D,N]    f32
    B: np.ndarray          # [b,L,G,N]
    C: np.ndarray          # [b,L,G,N]
    D: np.ndarray          # [D]      f32
    init: Optional[np.ndarray]  # [b,D,N] f32 or None

    @property
    def shape(self):
        b, L, Dc = self.x.shape
        return dict(b=b, L=L, D=Dc, G=self.B.shape[2], N=self.B.shape[3])

    def f64(self):
        """Exact float64 copies, in oracle argument order."""
        return dict(x=to_f64(self.x, self.dtype), dt=to_f64(self.dt, F32),
                    dt_bias=to_f64(self.dt_bias, F32), A=to_f64(self.A, F32),
                    B=to_f64(self.B, self.dtype), C=to_f64(self.C, self.dtype),
                    D=to_f64(self.D, F32),
                    init=None if self.init is None else to_f64(self.init, F32))


def make_sscan(b, L, Dc, G, N, *, dtype=BF16, seed=5, dt_range=(1e-3, 0.1),
               init_std: Optional[float] = None) -> SScanInputs:
    """A[d, n] = -(n + 1) * exp(U(-0.5, 0.5)): the real diagonal A = -(1..N)
    with a per-entry jitter, so that every (channel, n) has its own decay;
    per-channel step sizes exp(U(log dt_range)) through dt_bias =
    softplus^-1(dt); x ~ N(0,1); B, C ~ N(0,1)/sqrt(N); D ~ N(0,1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    A = -(np.arange(1, N + 1)[None, :] * np.exp(rng.uniform(-0.5, 0.5, size=(Dc, N))))
    dt_h = np.exp(rng.uniform(np.log(dt_range[0]), np.log(dt_range[1]), size=Dc))
    D = rng.standard_normal(Dc)
    x = rng.standard_normal((b, L, Dc))
    dt_raw = 0.5 * rng.standard_normal((b, L, Dc))
    Bm = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    Cm = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    init = None if init_std is None else init_std * rng.standard_normal((b, Dc, N))
    return SScanInputs(dtype=dtype, x=_store(x, dtype), dt=dt_raw.astype(np.float32),
                       dt_bias=_inv_softplus(dt_h).astype(np.float32), A=A.astype(np.float32),
                       B=_store(Bm, dtype), C=_store(Cm, dtype), D=D.astype(np.float32),
                       init=None if init is None else init.astype(np.float32))


# The selective-scan workload: a Mamba-1 2.8B layer (inner width 5120,
# N = 16) over 4 sequences of 2048 tokens.
SSCAN_WORKLOADS = {
    "mamba1_2p8b_b4_L2048_D5120_N16": dict(b=4, L=2048, Dc=5120, G=1, N=16, dtype=BF16, seed=5,
                                           init_std=0.1),
}


def make_sscan_workload(name: str) -> SScanInputs:
    w = dict(SSCAN_WORKLOADS[name])
    return make_sscan(w.pop("b"), w.pop("L"), w.pop("Dc"), w.pop("G"), w.pop("N"), **w)


def make_workload(name: str):
    w = dict(WORKLOADS[name])
    kind = w.pop("kind")
    if kind == "scan":
        return make_scan(w.pop("b"), w.pop("L"), w.pop("H"), w.pop("P"), w.pop("G"),
                         w.pop("N"), **w)
    return make_step(w.pop("b"), w.pop("H"), w.pop("P"), w.pop("G"), w.pop("N"),
                     w.pop("T"), **w)
