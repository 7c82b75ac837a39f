"""Gradients of the scan on the GPU (ssd_scan_bwd through the C ABI) against
the fp64 oracle's chain rule (oracle.scan_bwd), element by element.

Bound (every gradient): |got - ref| <= tol * (1 + |ref|), tol = 1e-4 for
fp32 inputs and 2e-2 for bf16 inputs, as for the forward scan.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_scan_05_amd import inputs, ssd, staging

pytestmark = pytest.mark.gpu
DEV = "cuda"
TOL = {inputs.F32: 1e-4, inputs.BF16: 2e-2}
NAMES = ["dx", "ddt", "dA", "dB", "dC", "ddt_bias", "dD", "dinit"]


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def check(got, ref, tol, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    den = 1.0 + np.abs(ref)
    err = float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0
    assert err <= tol, "%s: max |e|/(1+|ref|) = %.3e > %.1e" % (what, err, tol)
    return err


def make_grads_in(si, seed, dfinal=True):
    g = torch.Generator().manual_seed(seed)
    b, L, H, P = si.x.shape
    N = si.B.shape[3]
    dy = torch.randn((b, L, H, P), generator=g).to(torch.bfloat16 if si.dtype == inputs.BF16 else torch.float32)
    df = torch.randn((b, H, P, N), generator=g) if dfinal else None
    return dy, df


def run(si, dy, df, bias=True, skip=True, init=True):
    t = staging.scan_tensors(si, DEV)
    if not bias:
        t["dt_bias"] = None
    if not skip:
        t["D"] = None
    if not init:
        t["init_state"] = None
    g = ssd.ssd_scan_bwd(**t, dout=dy.to(DEV), dfinal_state=None if df is None else df.to(DEV),
                         want_dt_bias=bias, want_D=skip, want_init=True)
    torch.cuda.synchronize()
    return {k: (None if v is None else v.double().cpu().numpy()) for k, v in g.items()}


def ref_grads(si, dy, df, bias=True, skip=True, init=True):
    a = si.f64()
    return oracle.scan_bwd(a["x"], a["dt"], a["dt_bias"] if bias else None, a["A"], a["B"], a["C"],
                           a["D"] if skip else None, a["init"] if init else None,
                           dy.double().numpy(), None if df is None else df.double().numpy())


CASES = [
    # (b, L, H, P, G, N, dtype)
    (1, 64, 2, 32, 1, 32, inputs.F32),
    (2, 100, 4, 32, 2, 32, inputs.F32),
    (1, 300, 2, 64, 1, 64, inputs.F32),
    (2, 130, 2, 64, 2, 128, inputs.F32),
    (2, 200, 4, 64, 1, 128, inputs.BF16),
    (1, 257, 4, 32, 2, 128, inputs.BF16),
    (1, 1, 2, 32, 1, 64, inputs.F32),
    # P or N of 16 (run padded to 32 inside the chunk step)
    (1, 200, 4, 16, 1, 16, inputs.F32),
    (2, 130, 2, 16, 2, 64, inputs.BF16),
    (1, 100, 2, 32, 1, 16, inputs.BF16),
    (1, 257, 4, 64, 2, 16, inputs.F32),
]


@pytest.mark.parametrize("b,L,H,P,G,N,dtype", CASES, ids=["b%dL%dH%dP%dG%dN%d%s" % c for c in CASES])
@pytest.mark.parametrize("variant", ["full", "bare"])
def test_bwd_small(b, L, H, P, G, N, dtype, variant):
    full = variant == "full"
    say("bwd", b, L, H, P, G, N, dtype, variant)
    si = inputs.make_scan(b, L, H, P, G, N, dtype=dtype, seed=90 + L + N, init_std=0.3)
    dy, df = make_grads_in(si, 7 + L, dfinal=full)
    got = run(si, dy, df, bias=full, skip=full, init=full)
    ref = ref_grads(si, dy, df, bias=full, skip=full, init=full)
    tol = TOL[dtype]
    for k in NAMES:
        if got.get(k) is None:
            continue
        check(got[k], ref[k], tol, k)


def test_bwd_strong_decay_long():
    # 16 chunks; step sizes up to 8 so decays underflow inside a chunk
    si = inputs.make_scan(1, 1000, 2, 64, 1, 64, dtype=inputs.F32, seed=95, init_std=0.5,
                          dt_range=(0.5, 8.0))
    dy, df = make_grads_in(si, 96)
    say("bwd strong decay, L = 1000")
    got = run(si, dy, df)
    ref = ref_grads(si, dy, df)
    for k in NAMES:
        check(got[k], ref[k], 1e-4, k)


def test_bwd_deterministic():
    si = inputs.make_scan(2, 500, 8, 64, 2, 128, dtype=inputs.BF16, seed=97, init_std=0.3)
    dy, df = make_grads_in(si, 98)
    say("bwd twice, bitwise")
    a = run(si, dy, df)
    b = run(si, dy, df)
    for k in NAMES:
        assert np.array_equal(a[k], b[k]), k


def test_bwd_many_heads_one_group():
    # 80 heads share one B/C group: the chunk step accumulates dB and dC over
    # all 80 heads of the group in turn; every gradient against the full oracle
    si = inputs.make_scan(1, 1024, 80, 64, 1, 128, dtype=inputs.BF16, seed=131, init_std=0.1)
    dy, df = make_grads_in(si, 132)
    say("bwd b1 L1024 H80 G1 (80 heads per group), all gradients")
    got = run(si, dy, df)
    ref = ref_grads(si, dy, df)
    for k in NAMES:
        say("  %s %.3e" % (k, check(got[k], ref[k], 2e-2, k)))


def test_bwd_workload_2p7b_full():
    # the 2.7B layer shape (b=4, L=4096, H=80, P=64, G=1, N=128, bf16): every
    # gradient, dB and dC (sums over all 80 heads) included, against the full
    # fp64 oracle
    name = "mamba2_2p7b_b4_L4096_H80_P64_N128"
    si = inputs.make_workload(name)
    dy, df = make_grads_in(si, 99)
    say("bwd workload", name)
    got = run(si, dy, df)
    say("  oracle backward (full)")
    ref = ref_grads(si, dy, df)
    for k in NAMES:
        say("  %s %.3e" % (k, check(got[k], ref[k], 2e-2, k)))


@pytest.mark.parametrize("kind", ["frozen", "no_decay", "zero_x"])
def test_bwd_degenerate(kind):
    # frozen: Delta ~ 1e-13 (decays ~1, inputs barely enter, softplus' ~ Delta);
    # no_decay: A = 0 (every decay is 1); zero_x: x = 0 (only the initial state
    # reaches y, yet dx, dB, dDelta are nonzero)
    si = inputs.make_scan(2, 300, 4, 64, 2, 64, dtype=inputs.F32, seed=101, init_std=0.5)
    if kind == "frozen":
        si.dt[...] = -30.0
        si.dt_bias[...] = 0.0
    elif kind == "no_decay":
        si.A[...] = 0.0
        si.dt[...] = -3.0
    else:
        si.x[...] = 0
    dy, df = make_grads_in(si, 102)
    say("bwd degenerate", kind)
    got = run(si, dy, df)
    ref = ref_grads(si, dy, df)
    for k in NAMES:
        check(got[k], ref[k], 1e-4, "%s %s" % (kind, k))


GATED_CASES = [
    (2, 150, 4, 32, 2, 64, inputs.F32),
    (2, 300, 4, 64, 1, 128, inputs.BF16),
    (1, 70, 2, 16, 1, 16, inputs.BF16),
]


@pytest.mark.parametrize("b,L,H,P,G,N,dtype", GATED_CASES, ids=["b%dL%dH%dP%dG%dN%d%s" % c for c in GATED_CASES])
def test_bwd_gated(b, L, H, P, G, N, dtype):
    say("bwd gated", b, L, H, P, G, N, dtype)
    si = inputs.make_scan(b, L, H, P, G, N, dtype=dtype, seed=110 + L, init_std=0.3)
    z = inputs.make_gate(si, seed=111)
    dy, df = make_grads_in(si, 112)
    t = staging.scan_tensors(si, DEV)
    zt = staging.tensor(z, si.dtype, DEV)
    g = ssd.ssd_scan_bwd_gated(**t, z=zt, dout=dy.to(DEV), dfinal_state=df.to(DEV))
    torch.cuda.synchronize()
    got = {k: v.double().cpu().numpy() for k, v in g.items() if v is not None}
    a = si.f64()
    ref = oracle.scan_bwd_gated(a["x"], a["dt"], a["dt_bias"], a["A"], a["B"], a["C"], inputs.to_f64(z, si.dtype),
                                a["D"], a["init"], dy.double().numpy(), df.double().numpy())
    for k in NAMES + ["dz"]:
        check(got[k], ref[k], TOL[dtype], "gated " + k)


def test_bwd_long_sequence():
    # L = 2^18: 4096 chunks through both state walks
    si = inputs.make_scan(1, 1 << 18, 2, 32, 1, 32, dtype=inputs.BF16, seed=120, init_std=0.3)
    dy, df = make_grads_in(si, 121)
    say("bwd long sequence, L = 2^18")
    got = run(si, dy, df)
    ref = ref_grads(si, dy, df)
    for k in NAMES:
        check(got[k], ref[k], 2e-2, "long " + k)


def test_bwd_workload_long_gva_whole_group():
    # long GVA (b=1, L=65536, H=32, G=8): the state walks run in 8 segments.
    # One whole group (heads 0-3 with B/C group 0) and one head of another
    # group are cut out for the oracle: the gradients of a group's heads and
    # that group's dB, dC depend on nothing else
    name = "long_gva_b1_L65536_H32_G8_P64_N128"
    si = inputs.make_workload(name)
    if si.init is None:
        si.init = (0.3 * np.random.default_rng(122).standard_normal((1, 32, 64, 128))).astype(np.float32)
    dy, df = make_grads_in(si, 123)
    say("bwd workload", name)
    got = run(si, dy, df)
    H, G = si.x.shape[2], si.B.shape[2]
    a = si.f64()
    for heads in ([0, 1, 2, 3], [29]):
        groups = sorted({h * G // H for h in heads})
        ref = oracle.scan_bwd(a["x"][:, :, heads], a["dt"][:, :, heads], a["dt_bias"][heads], a["A"][heads],
                              a["B"][:, :, groups], a["C"][:, :, groups], a["D"][heads], a["init"][:, heads],
                              dy.double().numpy()[:, :, heads], df.double().numpy()[:, heads])
        check(got["dx"][:, :, heads], ref["dx"], 2e-2, "dx")
        check(got["ddt"][:, :, heads], ref["ddt"], 2e-2, "ddt")
        check(got["dinit"][:, heads], ref["dinit"], 2e-2, "dinit")
        for k in ("dA", "dD", "ddt_bias"):
            check(got[k][heads], ref[k], 2e-2, k)
        if len(heads) == H // G:  # a whole group: its dB, dC are complete
            check(got["dB"][:, :, groups], ref["dB"], 2e-2, "dB group %s" % groups)
            check(got["dC"][:, :, groups], ref["dC"], 2e-2, "dC group %s" % groups)
