"""Move host arrays from ``inputs`` to torch tensors (bf16 from uint16 bits)."""
from __future__ import annotations

import numpy as np
import torch

from .inputs import BF16, ScanInputs, SScanInputs, StepInputs


def tensor(a, dtype: str, device) -> torch.Tensor:
    if dtype == BF16:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
        return t.view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def scan_tensors(si: ScanInputs, device) -> dict:
    f = "f32"
    return dict(
        x=tensor(si.x, si.dtype, device), dt=tensor(si.dt, f, device),
        dt_bias=tensor(si.dt_bias, f, device), A=tensor(si.A, f, device),
        B=tensor(si.B, si.dtype, device), C=tensor(si.C, si.dtype, device),
        D=tensor(si.D, f, device),
        init_state=None if si.init is None else tensor(si.init, f, device))


def sscan_tensors(si: SScanInputs, device) -> dict:
    f = "f32"
    return dict(
        x=tensor(si.x, si.dtype, device), dt=tensor(si.dt, f, device),
        dt_bias=tensor(si.dt_bias, f, device), A=tensor(si.A, f, device),
        B=tensor(si.B, si.dtype, device), C=tensor(si.C, si.dtype, device),
        D=tensor(si.D, f, device),
        init_state=None if si.init is None else tensor(si.init, f, device))


def step_tensors(sp: StepInputs, device) -> dict:
    f = "f32"
    return dict(state=tensor(sp.state, f, device), x=tensor(sp.x, sp.dtype, device),
                dt=tensor(sp.delta, f, device), A=tensor(sp.A, f, device),
                B=tensor(sp.B, sp.dtype, device), C=tensor(sp.C, sp.dtype, device),
                D=tensor(sp.D, f, device))


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)
