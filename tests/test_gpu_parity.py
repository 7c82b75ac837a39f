"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Bound (elementwise, outputs and final states):
    |got - ref| <= tol * (1 + |ref|),  tol = 1e-4 for fp32 inputs,
                                       tol = 2e-2 for bf16 inputs.
The recurrent step with integer data, A = 0 and Delta = 1 must be bitwise
exact.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_scan_05_amd import inputs, ssd, staging

pytestmark = pytest.mark.gpu

TOL = {inputs.F32: 1e-4, inputs.BF16: 2e-2}
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def rel_err(got, ref):
    return float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref)))) if ref.size else 0.0


def check(got, ref, tol, what):
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % what
    err = rel_err(got, ref)
    assert err <= tol, "%s: max |e|/(1+|ref|) = %.3e > %.1e" % (what, err, tol)
    return err


def gpu_scan(si, algo=ssd.SSD_ALGO_AUTO, chunk=None, init=True):
    t = staging.scan_tensors(si, DEV)
    if not init:
        t["init_state"] = None
    out, fin = ssd.ssd_scan_fwd(**t, chunk=chunk or si.chunk, algo=algo)
    torch.cuda.synchronize()
    return staging.to_f64(out), staging.to_f64(fin)


def oracle_scan(si, init=True):
    f = si.f64()
    if not init:
        f["init"] = None
    return oracle.scan(**f)


# ---------------------------------------------------------------------------
# recurrent step

@pytest.mark.parametrize("dtype,N,vals", [(inputs.F32, 128, 3), (inputs.BF16, 16, 1)])
def test_step_exact_integers(dtype, N, vals):
    """A = 0, Delta = 1, small integers: every result is an exact integer."""
    rng = np.random.default_rng(5)
    b, H, P, G, T = 3, 8, 16, 2, 3
    say("step exact", dtype, N)
    state = rng.integers(-vals, vals + 1, (b, H, P, N)).astype(np.float32)
    st = torch.from_numpy(state).to(DEV)
    A = torch.zeros(H, device=DEV)
    D = torch.from_numpy(rng.integers(-vals, vals + 1, H).astype(np.float32)).to(DEV)
    dl = torch.ones(b, H, device=DEV)
    ref = state.astype(np.float64)
    for _ in range(T):
        x = rng.integers(-vals, vals + 1, (b, H, P)).astype(np.float32)
        Bm = rng.integers(-vals, vals + 1, (b, G, N)).astype(np.float32)
        Cm = rng.integers(-vals, vals + 1, (b, G, N)).astype(np.float32)
        cast = (lambda a: staging.tensor(inputs.f32_to_bf16_bits(a), dtype, DEV)) \
            if dtype == inputs.BF16 else (lambda a: staging.tensor(a, dtype, DEV))
        y = ssd.ssd_step(st, cast(x), dl, A, cast(Bm), cast(Cm), D)
        torch.cuda.synchronize()
        yr, ref = oracle.step(ref, x, np.ones((b, H)), np.zeros(H), Bm, Cm, D.cpu().numpy())
        assert np.array_equal(staging.to_f64(y), yr)
        assert np.array_equal(staging.to_f64(st), ref)


@pytest.mark.parametrize("dtype", [inputs.F32, inputs.BF16])
@pytest.mark.parametrize("N,G,P", [(16, 1, 16), (32, 2, 24), (64, 4, 64), (128, 1, 64), (256, 2, 8)])
def test_step_random(dtype, N, G, P):
    b, H, T = 5, 8, 4
    sp = inputs.make_step(b, H, P, G, N, T, dtype=dtype, seed=N + G)
    say("step random", dtype, N, G, P)
    t = staging.step_tensors(sp, DEV)
    ref = sp.state.astype(np.float64)
    for k in range(T):
        y = ssd.ssd_step(t["state"], t["x"][k], t["dt"][k], t["A"], t["B"][k], t["C"][k], t["D"])
        torch.cuda.synchronize()
        yr, ref = oracle.step(ref, inputs.to_f64(sp.x[k], dtype), sp.delta[k], sp.A,
                              inputs.to_f64(sp.B[k], dtype), inputs.to_f64(sp.C[k], dtype), sp.D)
        check(staging.to_f64(y), yr, TOL[dtype], "step y k=%d" % k)
        check(staging.to_f64(t["state"]), ref, TOL[dtype], "step state k=%d" % k)


# ---------------------------------------------------------------------------
# scan, small shapes spanning several sub-blocks, chunks and a ragged tail

SMALL = [
    # dtype, b, L, H, P, G, N, chunk
    (inputs.F32, 2, 200, 4, 16, 1, 16, 64),
    (inputs.F32, 1, 300, 2, 64, 2, 128, 128),
    (inputs.BF16, 2, 200, 4, 16, 2, 32, 64),
    (inputs.BF16, 1, 333, 4, 32, 4, 64, 128),
    (inputs.BF16, 2, 517, 4, 64, 1, 128, 256),
    (inputs.BF16, 1, 130, 2, 128, 1, 128, 64),
    (inputs.BF16, 1, 64, 3, 64, 3, 16, 64),
    (inputs.BF16, 1, 1, 2, 64, 1, 128, 256),
    (inputs.BF16, 1, 63, 2, 32, 1, 32, 64),
]


@pytest.mark.parametrize("algo", [ssd.SSD_ALGO_FUSED, ssd.SSD_ALGO_CHUNKED])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "%s-b%dL%dH%dP%dG%dN%dQ%d" % c)
def test_scan_small(case, algo):
    dtype, b, L, H, P, G, N, chunk = case
    si = inputs.make_scan(b, L, H, P, G, N, dtype=dtype, chunk=chunk, seed=L + P + N,
                          init_std=0.5)
    say("scan small", case, "algo", algo)
    y, fin = gpu_scan(si, algo=algo)
    yr, fr = oracle_scan(si)
    check(y, yr, TOL[dtype], "y")
    check(fin, fr, TOL[dtype], "final_state")


@pytest.mark.parametrize("algo", [ssd.SSD_ALGO_FUSED, ssd.SSD_ALGO_CHUNKED])
def test_scan_zero_init_and_no_optional(algo):
    si = inputs.make_scan(2, 150, 4, 64, 2, 64, dtype=inputs.BF16, chunk=64, seed=9)
    say("scan no-optional algo", algo)
    t = staging.scan_tensors(si, DEV)
    out, _ = ssd.ssd_scan_fwd(t["x"], t["dt"], None, t["A"], t["B"], t["C"], None, None,
                              chunk=64, algo=algo, return_final_state=False)
    torch.cuda.synchronize()
    f = si.f64()
    yr, _ = oracle.scan(f["x"], f["dt"], None, f["A"], f["B"], f["C"], None, None)
    check(staging.to_f64(out), yr, 2e-2, "y without bias/D/init")


# ---------------------------------------------------------------------------
# the named workloads at full size, in the launch configuration the
# benchmark uses (automatic algorithm choice), and the other algorithm

SCANS = [n for n in inputs.WORKLOAD_ORDER if inputs.WORKLOADS[n]["kind"] == "scan"]
_CACHE = {}


def workload_with_reference(name):
    """Inputs and oracle outputs of a named workload, computed once."""
    if name not in _CACHE:
        _CACHE.clear()
        si = inputs.make_workload(name)
        _CACHE[name] = (si, oracle_scan(si))
    return _CACHE[name]


@pytest.mark.parametrize("algo", [ssd.SSD_ALGO_AUTO, ssd.SSD_ALGO_FUSED, ssd.SSD_ALGO_CHUNKED,
                                  ssd.SSD_ALGO_ROWS])
@pytest.mark.parametrize("name", SCANS)
def test_workload_scan(name, algo):
    if name.startswith("long") and algo == ssd.SSD_ALGO_FUSED:
        pytest.skip("one workgroup per (batch, head) leaves most of the GPU idle here; "
                    "covered by the small-shape tests")
    if algo == ssd.SSD_ALGO_ROWS and inputs.WORKLOADS[name]["dtype"] != inputs.BF16:
        pytest.skip("the row-sliced walk takes bf16 inputs only")
    say("workload", name, "algo", algo)
    si, (yr, fr) = workload_with_reference(name)
    y, fin = gpu_scan(si, algo=algo)
    ey = check(y, yr, TOL[si.dtype], "%s y" % name)
    ef = check(fin, fr, TOL[si.dtype], "%s final" % name)
    say("  max rel err y %.3e final %.3e" % (ey, ef))


def test_workload_decode_steps():
    name = "decode_step_b256_H80_P64_N128_T64"
    sp = inputs.make_workload(name)
    say("workload", name)
    t = staging.step_tensors(sp, DEV)
    ref = sp.state.astype(np.float64)
    T = sp.x.shape[0]
    sb_idx = torch.as_tensor(SAMPLE_B, device=DEV)
    sh_idx = torch.as_tensor(SAMPLE_H, device=DEV)
    worst = 0.0
    for k in range(T):
        y = ssd.ssd_step(t["state"], t["x"][k], t["dt"][k], t["A"], t["B"][k], t["C"][k], t["D"])
        yr, ref = oracle.step(ref, inputs.to_f64(sp.x[k], sp.dtype), sp.delta[k], sp.A,
                              inputs.to_f64(sp.B[k], sp.dtype), inputs.to_f64(sp.C[k], sp.dtype),
                              sp.D)
        worst = max(worst, check(staging.to_f64(y), yr, 2e-2, "decode y step %d" % k))
        # the state after this step on a fixed sample of (batch, head) slices
        got_s = t["state"][sb_idx, sh_idx].cpu().numpy().astype(np.float64)
        worst = max(worst, check(got_s, ref[SAMPLE_B, SAMPLE_H], 2e-2, "decode state step %d" % k))
    torch.cuda.synchronize()
    worst = max(worst, check(staging.to_f64(t["state"]), ref, 2e-2, "decode state"))
    say("  max rel err %.3e" % worst)


# (batch, head) slices of the decode state compared after every step: the
# first and last batch rows and heads plus a spread of others
SAMPLE_B = np.array([0, 255, 1, 37, 128, 200, 77, 254, 3, 160, 99, 31])
SAMPLE_H = np.array([0, 79, 40, 1, 63, 17, 78, 5, 33, 50, 71, 12])


def test_exported_scan_fwd_symbol():
    """ssd_scan_fwd itself (not the algorithm-selecting variant), called through
    ctypes with hand-built descriptors and the raw stream handle."""
    import ctypes
    si = inputs.make_scan(2, 300, 8, 64, 2, 128, dtype=inputs.BF16, seed=31, init_std=0.1)
    t = staging.scan_tensors(si, DEV)
    b, L, H, P = si.x.shape
    N = si.B.shape[3]
    out = torch.empty_like(t["x"])
    fin = torch.full((b, H, P, N), float("nan"), dtype=torch.float32, device=DEV)
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    say("ssd_scan_fwd symbol")
    lib = ssd.lib()
    fn = lib.ssd_scan_fwd
    assert fn.argtypes[-2] is ctypes.c_int and len(fn.argtypes) == 12
    status = fn(ssd.describe(t["x"]), ssd.describe(t["dt"]), ssd.describe(t["dt_bias"]),
                ssd.describe(t["A"]), ssd.describe(t["B"]), ssd.describe(t["C"]), ssd.describe(t["D"]),
                ssd.describe(t["init_state"]), ssd.describe(out), ssd.describe(fin), 256,
                ctypes.c_void_p(stream.cuda_stream))
    assert status == 0, lib.ssd_last_error().decode()
    stream.synchronize()
    yr, fr = oracle_scan(si)
    check(staging.to_f64(out), yr, 2e-2, "ssd_scan_fwd y")
    check(staging.to_f64(fin), fr, 2e-2, "ssd_scan_fwd final")
    # a rejected call returns its status before any launch
    bad = fn(ssd.describe(t["x"]), ssd.describe(t["dt"]), None, ssd.describe(t["A"]),
             ssd.describe(t["B"]), ssd.describe(t["C"]), None, None, ssd.describe(out), None, 100,
             ctypes.c_void_p(stream.cuda_stream))
    assert bad == 5 and b"chunk" in lib.ssd_last_error()


# ---------------------------------------------------------------------------
# invariants on the device

def test_chunk_invariance():
    si = inputs.make_scan(2, 1000, 8, 64, 2, 128, dtype=inputs.BF16, seed=21, init_std=0.1)
    outs = []
    for chunk in (64, 128, 256, 512, 1024, 4096):
        say("chunk invariance", chunk)
        outs.append(gpu_scan(si, algo=ssd.SSD_ALGO_CHUNKED, chunk=chunk))
    outs.append(gpu_scan(si, algo=ssd.SSD_ALGO_FUSED))
    outs.append(gpu_scan(si, algo=ssd.SSD_ALGO_ROWS))
    yr, fr = oracle_scan(si)
    check(outs[0][0], yr, 2e-2, "y chunk 64")
    check(outs[0][1], fr, 2e-2, "final chunk 64")
    for y, f in outs[1:]:
        check(y, outs[0][0], 2e-2, "y across chunk sizes")
        check(f, outs[0][1], 2e-2, "final across chunk sizes")


@pytest.mark.parametrize("algo", [ssd.SSD_ALGO_FUSED, ssd.SSD_ALGO_CHUNKED, ssd.SSD_ALGO_ROWS])
@pytest.mark.parametrize("L1", [256, 300])
def test_split_invariance(algo, L1):
    """Scanning [0, L1) then [L1, L) from the carried state equals one scan."""
    si = inputs.make_scan(2, 700, 4, 64, 1, 128, dtype=inputs.BF16, seed=22, init_std=0.1)
    say("split", algo, L1)
    t = staging.scan_tensors(si, DEV)
    y, f = ssd.ssd_scan_fwd(**t, chunk=256, algo=algo)
    a = {k: v for k, v in t.items()}
    for k in ("x", "dt", "B", "C"):
        a[k] = t[k][:, :L1].contiguous()
    y1, f1 = ssd.ssd_scan_fwd(**a, chunk=256, algo=algo)
    for k in ("x", "dt", "B", "C"):
        a[k] = t[k][:, L1:].contiguous()
    a["init_state"] = f1
    y2, f2 = ssd.ssd_scan_fwd(**a, chunk=256, algo=algo)
    torch.cuda.synchronize()
    check(staging.to_f64(torch.cat([y1, y2], 1)), staging.to_f64(y), 2e-2, "split y")
    check(staging.to_f64(f2), staging.to_f64(f), 2e-2, "split final")


def test_in_place_final_state():
    si = inputs.make_scan(1, 300, 4, 64, 1, 64, dtype=inputs.BF16, seed=23, init_std=0.3)
    say("in-place final state")
    t = staging.scan_tensors(si, DEV)
    st = t["init_state"].clone()
    for algo in (ssd.SSD_ALGO_FUSED, ssd.SSD_ALGO_CHUNKED, ssd.SSD_ALGO_ROWS):
        t2 = dict(t, init_state=st.clone())
        ssd.ssd_scan_fwd(**dict(t2, final_state=t2["init_state"]), chunk=64, algo=algo)
        torch.cuda.synchronize()
        _, fr = oracle_scan(si)
        check(staging.to_f64(t2["init_state"]), fr, 2e-2, "in-place final algo %d" % algo)


def test_step_matches_scan():
    si = inputs.make_scan(2, 40, 4, 64, 2, 128, dtype=inputs.F32, seed=24, init_std=0.2)
    say("step vs scan")
    t = staging.scan_tensors(si, DEV)
    y, f = ssd.ssd_scan_fwd(**t, chunk=64, algo=ssd.SSD_ALGO_FUSED)
    delta = torch.nn.functional.softplus(t["dt"].double() + t["dt_bias"].double()).float()
    st = t["init_state"].clone()
    for k in range(si.x.shape[1]):
        yk = ssd.ssd_step(st, t["x"][:, k].contiguous(), delta[:, k].contiguous(), t["A"],
                          t["B"][:, k].contiguous(), t["C"][:, k].contiguous(), t["D"])
        check(staging.to_f64(yk), staging.to_f64(y[:, k]), 1e-4, "step %d vs scan" % k)
    torch.cuda.synchronize()
    check(staging.to_f64(st), staging.to_f64(f), 1e-4, "step state vs scan final")


@pytest.mark.parametrize("algo", [ssd.SSD_ALGO_FUSED, ssd.SSD_ALGO_CHUNKED, ssd.SSD_ALGO_ROWS])
def test_deterministic(algo):
    si = inputs.make_scan(2, 777, 8, 64, 1, 128, dtype=inputs.BF16, seed=25, init_std=0.1)
    say("determinism", algo)
    t = staging.scan_tensors(si, DEV)
    y1, f1 = ssd.ssd_scan_fwd(**t, chunk=256, algo=algo)
    y2, f2 = ssd.ssd_scan_fwd(**t, chunk=256, algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(f1, f2)


@pytest.mark.parametrize("chunk", [512, 2048])
def test_long_segments_ragged(chunk):
    """Segments of many sub-blocks with a ragged last segment."""
    si = inputs.make_scan(1, 2 * chunk + 333, 4, 64, 2, 128, dtype=inputs.BF16, seed=chunk,
                          init_std=0.2)
    say("long segments", chunk)
    y, fin = gpu_scan(si, algo=ssd.SSD_ALGO_CHUNKED, chunk=chunk)
    yr, fr = oracle_scan(si)
    check(y, yr, 2e-2, "y")
    check(fin, fr, 2e-2, "final")


# ---------------------------------------------------------------------------
# the row-sliced walk (bf16, N in {32, 64, 128}) at every workgroup size

ROWS_SMALL = [c for c in SMALL if c[0] == inputs.BF16 and c[6] in (32, 64, 128)] + [
    # heads per group not a multiple of the workgroup's rows; idle waves
    (inputs.BF16, 2, 300, 6, 32, 2, 64, 64),
    (inputs.BF16, 1, 200, 12, 16, 3, 128, 64),
    (inputs.BF16, 3, 129, 5, 64, 5, 32, 64),
    # more than 128 heads: the head-major step-size copy takes two passes
    # (H a multiple of 4: 16-byte reads; H = 130: element reads)
    (inputs.BF16, 1, 150, 136, 16, 1, 32, 64),
    (inputs.BF16, 2, 70, 130, 16, 2, 32, 64),
]


@pytest.mark.parametrize("waves", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("case", ROWS_SMALL, ids=lambda c: "%s-b%dL%dH%dP%dG%dN%dQ%d" % c)
def test_rows_small(case, waves):
    dtype, b, L, H, P, G, N, chunk = case
    si = inputs.make_scan(b, L, H, P, G, N, dtype=dtype, chunk=chunk, seed=L + P + N + 1,
                          init_std=0.5)
    say("rows small", case, "waves", waves)
    t = staging.scan_tensors(si, DEV)
    out, fin = ssd.ssd_scan_fwd_rows(**t, waves=waves)
    torch.cuda.synchronize()
    yr, fr = oracle_scan(si)
    check(staging.to_f64(out), yr, TOL[dtype], "y")
    check(staging.to_f64(fin), fr, TOL[dtype], "final_state")


def decay_spans(si):
    """|sum of Delta*A*log2(e)| over each 64-token sub-block, per (b, h)."""
    f = si.f64()
    dl = np.logaddexp(0.0, f["dt"] + f["dt_bias"][None, None, :])
    a = np.abs(dl * f["A"][None, None, :]) * np.log2(np.e)
    b, L, H = a.shape
    pad = (-L) % 64
    a = np.concatenate([a, np.zeros((b, pad, H))], 1)
    return a.reshape(b, -1, 64, H).sum(2)


@pytest.mark.parametrize("waves", [1, 4, 5])
def test_rows_strong_decay(waves):
    """Sub-blocks whose decay span exceeds the separable range (per-element
    path, span > 178 log2 units) next to wide separable ones (90 < span <=
    178, renormalised every sub-block) and ordinary ones, in the same
    workgroups."""
    si = inputs.make_scan(2, 300, 8, 64, 2, 128, dtype=inputs.BF16, seed=31,
                          dt_range=(0.01, 2.0), init_std=0.3)
    spans = decay_spans(si)
    assert (spans > 178).any() and ((spans > 90) & (spans <= 178)).any() and (spans <= 90).any()
    say("rows strong decay waves", waves, "slow share %.2f" % float((spans > 178).mean()))
    t = staging.scan_tensors(si, DEV)
    out, fin = ssd.ssd_scan_fwd_rows(**t, waves=waves)
    torch.cuda.synchronize()
    yr, fr = oracle_scan(si)
    check(staging.to_f64(out), yr, 2e-2, "y")
    check(staging.to_f64(fin), fr, 2e-2, "final_state")


@pytest.mark.parametrize("waves", [1, 4, 5])
def test_rows_exponent_renormalisation(waves):
    """32 sub-blocks per head with decay spans from 34 to 183 log2 units: the
    running state exponent is renormalised many times, one head alternates
    between the separable and the per-element path, and the final state
    carries the accumulated exponent."""
    si = inputs.make_scan(1, 2048, 4, 64, 1, 64, dtype=inputs.BF16, seed=37,
                          dt_range=(0.03, 0.4), A_range=(4.0, 16.0), init_std=0.3)
    spans = decay_spans(si)
    assert (spans > 178).any() and ((spans > 90) & (spans <= 178)).mean() > 0.3
    say("rows exponent renormalisation waves", waves)
    t = staging.scan_tensors(si, DEV)
    out, fin = ssd.ssd_scan_fwd_rows(**t, waves=waves)
    torch.cuda.synchronize()
    yr, fr = oracle_scan(si)
    check(staging.to_f64(out), yr, 2e-2, "y")
    check(staging.to_f64(fin), fr, 2e-2, "final_state")


def test_rows_no_optional():
    si = inputs.make_scan(2, 150, 4, 64, 2, 64, dtype=inputs.BF16, chunk=64, seed=9)
    say("rows no-optional")
    t = staging.scan_tensors(si, DEV)
    out, _ = ssd.ssd_scan_fwd_rows(t["x"], t["dt"], None, t["A"], t["B"], t["C"], None, None,
                                   waves=2, return_final_state=False)
    torch.cuda.synchronize()
    f = si.f64()
    yr, _ = oracle.scan(f["x"], f["dt"], None, f["A"], f["B"], f["C"], None, None)
    check(staging.to_f64(out), yr, 2e-2, "y without bias/D/init")


def test_rows_waves_agree():
    """Every state row is computed by the same instructions whatever the
    workgroup size, so outputs agree bitwise across wave counts."""
    si = inputs.make_scan(2, 400, 10, 64, 1, 128, dtype=inputs.BF16, seed=33, init_std=0.2)
    t = staging.scan_tensors(si, DEV)
    ref = None
    for waves in range(1, 9):
        say("rows waves agree", waves)
        out, fin = ssd.ssd_scan_fwd_rows(**t, waves=waves)
        torch.cuda.synchronize()
        if ref is None:
            ref = (out.clone(), fin.clone())
        else:
            assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), waves
            assert torch.equal(fin, ref[1]), waves


# ---------------------------------------------------------------------------
# the gated output out = y * silu(z), every algorithm

def gated_case(si, seed):
    z = inputs.make_gate(si, seed=seed)
    return z, inputs.to_f64(z, si.dtype)


def oracle_scan_gated(si, zf):
    f = si.f64()
    return oracle.scan_gated(f["x"], f["dt"], f["dt_bias"], f["A"], f["B"], f["C"], zf, f["D"], f["init"])


GATED = [
    # dtype, b, L, H, P, G, N, chunk
    (inputs.F32, 1, 300, 2, 64, 2, 128, 128),
    (inputs.F32, 2, 200, 4, 16, 1, 16, 64),
    (inputs.BF16, 2, 517, 4, 64, 1, 128, 256),
    (inputs.BF16, 1, 333, 4, 32, 4, 64, 128),
]


@pytest.mark.parametrize("algo", [ssd.SSD_ALGO_FUSED, ssd.SSD_ALGO_CHUNKED, ssd.SSD_ALGO_ROWS])
@pytest.mark.parametrize("case", GATED, ids=lambda c: "%s-b%dL%dH%dP%dG%dN%dQ%d" % c)
def test_gated_small(case, algo):
    dtype, b, L, H, P, G, N, chunk = case
    if algo == ssd.SSD_ALGO_ROWS and (dtype != inputs.BF16 or N == 16):
        pytest.skip("the row-sliced walk takes bf16 inputs and N >= 32")
    si = inputs.make_scan(b, L, H, P, G, N, dtype=dtype, chunk=chunk, seed=L + P + N + 7,
                          init_std=0.5)
    z, zf = gated_case(si, seed=L + 3)
    say("gated small", case, "algo", algo)
    t = staging.scan_tensors(si, DEV)
    out, fin = ssd.ssd_scan_fwd_gated(**t, z=staging.tensor(z, dtype, DEV), chunk=chunk, algo=algo)
    torch.cuda.synchronize()
    yr, fr = oracle_scan_gated(si, zf)
    check(staging.to_f64(out), yr, TOL[dtype], "gated y")
    check(staging.to_f64(fin), fr, TOL[dtype], "final_state")


# Shapes whose automatic workgroup size on a 256-unit MI355X is 1, 5 and 8
# waves: the direct-store schedule and the staged-store schedule.
GATED_ROWS = [
    (3, 129, 5, 64, 5, 32),     # 1 wave per workgroup, idle rows, ragged tail
    (4, 300, 80, 64, 1, 128),   # 5 waves
    (4, 200, 128, 64, 1, 128),  # 8 waves
]


@pytest.mark.parametrize("case", GATED_ROWS, ids=lambda c: "b%dL%dH%dP%dG%dN%d" % c)
def test_gated_rows_schedules(case):
    b, L, H, P, G, N = case
    si = inputs.make_scan(b, L, H, P, G, N, dtype=inputs.BF16, chunk=64, seed=41 + H, init_std=0.5)
    z, zf = gated_case(si, seed=42 + H)
    say("gated rows", case)
    t = staging.scan_tensors(si, DEV)
    out, fin = ssd.ssd_scan_fwd_gated(**t, z=staging.tensor(z, inputs.BF16, DEV), chunk=64,
                                      algo=ssd.SSD_ALGO_ROWS)
    torch.cuda.synchronize()
    yr, fr = oracle_scan_gated(si, zf)
    check(staging.to_f64(out), yr, 2e-2, "gated y")
    check(staging.to_f64(fin), fr, 2e-2, "final_state")


def test_gated_workload_2p7b():
    """The 2.7B layer shape at full size, automatic plan (the benchmark's)."""
    si, _ = workload_with_reference("mamba2_2p7b_b4_L4096_H80_P64_N128")
    z, zf = gated_case(si, seed=5)
    say("gated workload 2.7B")
    t = staging.scan_tensors(si, DEV)
    out, fin = ssd.ssd_scan_fwd_gated(**t, z=staging.tensor(z, si.dtype, DEV), chunk=si.chunk)
    torch.cuda.synchronize()
    yr, fr = oracle_scan_gated(si, zf)
    ey = check(staging.to_f64(out), yr, 2e-2, "gated y")
    ef = check(staging.to_f64(fin), fr, 2e-2, "final_state")
    say("  max rel err y %.3e final %.3e" % (ey, ef))


def test_host_memory_refused_on_device():
    # pageable host tensors, alone or mixed with device tensors, are refused
    # on the host before any launch
    b, L, H, P, G, N = 1, 100, 4, 16, 2, 32
    bf = torch.bfloat16

    def args(dev, B_dev):
        return dict(x=torch.zeros(b, L, H, P, dtype=bf, device=dev), dt=torch.zeros(b, L, H, device=dev),
                    dt_bias=torch.zeros(H, device=dev), A=-torch.ones(H, device=dev),
                    B=torch.zeros(b, L, G, N, dtype=bf, device=B_dev),
                    C=torch.zeros(b, L, G, N, dtype=bf, device=dev), D=torch.zeros(H, device=dev))
    say("host memory refusal: all on the host, then B on the host")
    for dev, B_dev, culprit in (("cpu", "cpu", "x"), (DEV, "cpu", "B")):
        a = args(dev, B_dev)
        out = torch.zeros(b, L, H, P, dtype=bf, device=dev)
        with pytest.raises(ssd.SsdError) as e:
            ssd.ssd_scan_fwd(**a, out=out, return_final_state=False, chunk=64)
        assert e.value.status == 4, str(e.value)
        assert ("%s:" % culprit) in str(e.value), str(e.value)
    torch.cuda.synchronize()
