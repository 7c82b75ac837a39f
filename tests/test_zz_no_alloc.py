"""The allocation-free entry point ssd_scan_fwd_noalloc (scratch in the
library's fixed device array) against ssd_scan_fwd, through the C ABI: two
calls in a row, the second with a smaller input, each bitwise equal to
ssd_scan_fwd on the same inputs and within the bf16 bound of the fp64 oracle.
A plan that needs more scratch than the fixed array holds is refused."""
import sys

import numpy as np
import pytest
import torch

import oracle
from mamba_ssd_scan_05_amd import inputs, ssd, staging

pytestmark = pytest.mark.gpu
DEV = "cuda"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run_pair(si):
    t = staging.scan_tensors(si, DEV)
    b, L, H, P = si.x.shape
    N = si.B.shape[3]
    ref_out, ref_fin = ssd.ssd_scan_fwd(**t, chunk=si.chunk)
    out = torch.full_like(t["x"], float("nan"))
    fin = torch.full((b, H, P, N), float("nan"), dtype=torch.float32, device=DEV)
    ssd.ssd_scan_fwd_noalloc(**t, out=out, final_state=fin, chunk=si.chunk)
    torch.cuda.synchronize()
    return (staging.to_f64(out), staging.to_f64(fin)), (staging.to_f64(ref_out), staging.to_f64(ref_fin))


def check_against(got, ref, si):
    yr, fr = oracle.scan(**si.f64())
    for g, r, o, what in ((got[0], ref[0], yr, "y"), (got[1], ref[1], fr, "final")):
        assert np.array_equal(g, r), "%s differs from ssd_scan_fwd" % what
        err = float(np.max(np.abs(g - o) / (1 + np.abs(o))))
        assert err <= 2e-2, "%s: %.3e" % (what, err)


def test_noalloc_two_calls_second_smaller():
    big = inputs.make_scan(2, 4096, 80, 64, 1, 128, dtype=inputs.BF16, seed=141, init_std=0.1)
    small = inputs.make_scan(1, 300, 8, 64, 2, 128, dtype=inputs.BF16, seed=142, init_std=0.1)
    for name, si in (("big", big), ("small", small)):
        say("noalloc", name, si.x.shape)
        got, ref = run_pair(si)
        check_against(got, ref, si)


def test_noalloc_chunked_plan_and_fp32():
    # the long, narrow shape takes the chunked plan (segment states in the
    # fixed array); fp32 takes a walk of its own
    cases = [inputs.make_scan(1, 16384, 4, 64, 1, 64, dtype=inputs.BF16, seed=143, init_std=0.2),
             inputs.make_scan(1, 1000, 4, 32, 1, 32, dtype=inputs.F32, seed=144, init_std=0.2)]
    for si in cases:
        say("noalloc", si.x.shape, si.dtype)
        got, ref = run_pair(si)
        if si.dtype == inputs.F32:
            yr, fr = oracle.scan(**si.f64())
            assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
            assert float(np.max(np.abs(got[0] - yr) / (1 + np.abs(yr)))) <= 1e-4
        else:
            check_against(got, ref, si)


def test_noalloc_refuses_scratch_above_the_fixed_array():
    # a long sequence over few (batch, head) pairs takes the chunked plan,
    # whose step sizes alone are b*H*L*4 bytes (here 256 MiB): refused with
    # SSD_ERR_NOMEM before any launch, and the output is left untouched
    b, L, H, P, G, N = 1, 1 << 20, 64, 16, 8, 32
    x = torch.zeros(b, L, H, P, dtype=torch.bfloat16, device=DEV)
    Bm = torch.zeros(b, L, G, N, dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(x, 7.0)
    args = dict(x=x, dt=torch.zeros(b, L, H, device=DEV), dt_bias=None, A=-torch.ones(H, device=DEV),
                B=Bm, C=Bm.clone(), D=None, init_state=None, out=out, final_state=None)
    a, seg = ssd.ssd_scan_plan(b, L, H, P, G, N, torch.bfloat16, 256)
    assert a == ssd.SSD_ALGO_CHUNKED, (a, seg)
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_scan_fwd_noalloc(**args)
    torch.cuda.synchronize()
    assert e.value.status == 7 and "fixed scratch" in str(e.value), str(e.value)
    assert bool(torch.all(out == 7.0))
