"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects invalid arguments before any HIP call (CPU only)."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def ssd():
    from mamba_ssd_scan_05_amd import ssd as mod
    if not os.path.exists(mod.LIB_PATH):
        from mamba_ssd_scan_05_amd import build
        build.build()
    return mod


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ssd_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(ssd):
    names = declared_functions()
    assert {"ssd_scan_fwd", "ssd_step", "ssd_scan_fwd_algo", "ssd_scan_fwd_rows", "ssd_scan_fwd_gated",
            "ssd_selective_scan_fwd",
            "ssd_scan_plan", "ssd_status_string", "ssd_last_error", "ssd_version",
            "ssd_release_scratch"} <= set(names)
    raw = ctypes.CDLL(ssd.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    out = os.popen("nm -D --defined-only %s" % ssd.LIB_PATH).read()
    for n in names:
        assert re.search(r"\bT %s\b" % n, out), n


def test_release_scratch_with_nothing_kept(ssd):
    # no call has taken scratch in this process: nothing to free, no HIP call
    assert ssd.lib().ssd_release_scratch() == 0
    ssd.ssd_release_scratch()


def test_scratch_stats_host_only(ssd):
    # nothing kept in this process: zero buffers, zero bytes; NULL refused
    assert ssd.ssd_scratch_stats() == (0, 0)
    assert ssd.lib().ssd_scratch_stats(None, None) == 1
    assert ssd.ssd_fixed_scratch_bytes() == 64 << 20


def test_version_and_strings(ssd):
    assert ssd.ssd_version() == 100
    assert ssd.ssd_status_string(0) == "ok"
    assert ssd.ssd_status_string(6) == "output aliases an input"
    assert ssd.ssd_status_string(1234) == "unknown status"


def _scan_args(b=1, L=100, H=4, P=16, G=2, N=32, dtype=torch.bfloat16):
    return dict(x=torch.zeros(b, L, H, P, dtype=dtype), dt=torch.zeros(b, L, H),
                dt_bias=torch.zeros(H), A=-torch.ones(H), B=torch.zeros(b, L, G, N, dtype=dtype),
                C=torch.zeros(b, L, G, N, dtype=dtype), D=torch.zeros(H),
                init_state=torch.zeros(b, H, P, N), out=torch.zeros(b, L, H, P, dtype=dtype),
                final_state=torch.zeros(b, H, P, N))


def _call_scan(ssd, a, chunk=64, algo=0):
    lib = ssd.lib()
    d = ssd.describe
    st = lib.ssd_scan_fwd_algo(d(a["x"]), d(a["dt"]), d(a["dt_bias"]), d(a["A"]), d(a["B"]),
                               d(a["C"]), d(a["D"]), d(a["init_state"]), d(a["out"]),
                               d(a["final_state"]), chunk, algo, None)
    return st, ssd.ssd_last_error()


CASES = [
    ("x_none", lambda a: a.update(x=None), 1),
    ("A_none", lambda a: a.update(A=None), 1),
    ("out_none", lambda a: a.update(out=None), 1),
    ("L_zero", lambda a: a.update(x=torch.zeros(1, 0, 4, 16, dtype=torch.bfloat16)), 2),
    ("H_not_multiple_of_G", lambda a: a.update(B=torch.zeros(1, 100, 3, 32, dtype=torch.bfloat16),
                                               C=torch.zeros(1, 100, 3, 32, dtype=torch.bfloat16)), 2),
    ("dt_wrong_shape", lambda a: a.update(dt=torch.zeros(1, 99, 4)), 2),
    ("C_wrong_N", lambda a: a.update(C=torch.zeros(1, 100, 2, 16, dtype=torch.bfloat16)), 2),
    ("init_wrong_shape", lambda a: a.update(init_state=torch.zeros(1, 4, 16, 16)), 2),
    ("dt_bf16", lambda a: a.update(dt=torch.zeros(1, 100, 4, dtype=torch.bfloat16)), 3),
    ("B_f32_with_bf16_x", lambda a: a.update(B=torch.zeros(1, 100, 2, 32)), 3),
    ("x_f16", lambda a: a.update(x=torch.zeros(1, 100, 4, 16, dtype=torch.float16)), 3),
    ("out_f32", lambda a: a.update(out=torch.zeros(1, 100, 4, 16)), 3),
    ("x_noncontiguous", lambda a: a.update(
        x=torch.zeros(1, 4, 100, 16, dtype=torch.bfloat16).transpose(1, 2)), 4),
    ("x_misaligned", lambda a: a.update(
        x=torch.zeros(1 * 100 * 4 * 16 + 1, dtype=torch.bfloat16)[1:].view(1, 100, 4, 16)), 4),
    ("P_unsupported", lambda a: a.update(x=torch.zeros(1, 100, 4, 24, dtype=torch.bfloat16),
                                         out=torch.zeros(1, 100, 4, 24, dtype=torch.bfloat16)), 5),
    ("P128_fp32_unsupported", lambda a: a.update(
        x=torch.zeros(1, 100, 4, 128), out=torch.zeros(1, 100, 4, 128),
        B=torch.zeros(1, 100, 2, 32), C=torch.zeros(1, 100, 2, 32),
        init_state=torch.zeros(1, 4, 128, 32), final_state=torch.zeros(1, 4, 128, 32)), 5),
    ("N_unsupported", lambda a: a.update(B=torch.zeros(1, 100, 2, 48, dtype=torch.bfloat16),
                                         C=torch.zeros(1, 100, 2, 48, dtype=torch.bfloat16)), 5),
]


def _fake(ssd, shape, dtype, slot=0):
    """A descriptor of a dense tensor at a fake aligned address (validation
    only reads the descriptor); distinct slots do not overlap."""
    t = ssd.SsdTensor()
    t.data = (1 << 20) + slot * (1 << 44)
    t.dtype = dtype
    t.ndim = len(shape)
    st = 1
    for i in range(len(shape) - 1, -1, -1):
        t.shape[i] = shape[i]
        t.strides[i] = st
        st *= shape[i]
    return t


@pytest.mark.parametrize("b,L,H,P,G,N", [(1, (1 << 24) + 64, 1, 16, 1, 16),
                                         (1, 64, (1 << 18) + 1, 16, 1, 16),
                                         (1, 64, 1 << 16, 16, 1 << 16, 128)],
                         ids=["L_above_max", "HP_above_max", "GN_above_max"])
def test_scan_rejects_oversized(ssd, b, L, H, P, G, N):
    # shapes whose per-tile byte ranges would not fit 32 bits are refused
    # on the host before any device call
    bf, f32 = 1, 0
    x = _fake(ssd, (b, L, H, P), bf)
    args = [x, _fake(ssd, (b, L, H), f32), None, _fake(ssd, (H,), f32),
            _fake(ssd, (b, L, G, N), bf), _fake(ssd, (b, L, G, N), bf), None, None,
            _fake(ssd, (b, L, H, P), bf), None]
    lib = ssd.lib()
    P_ = ctypes.POINTER(ssd.SsdTensor)
    ptrs = [ctypes.byref(a) if a is not None else None for a in args]
    st = lib.ssd_scan_fwd_algo(*ptrs, 256, 0, None)
    assert st == 5, (st, ssd.ssd_last_error())
    assert "supported" in ssd.ssd_last_error()


@pytest.mark.parametrize("name,mutate,status", CASES, ids=[c[0] for c in CASES])
def test_scan_rejects(ssd, name, mutate, status):
    a = _scan_args()
    mutate(a)
    st, msg = _call_scan(ssd, a)
    assert st == status, (st, msg)
    assert msg


def test_scan_rejects_bad_chunk_and_algo(ssd):
    a = _scan_args()
    assert _call_scan(ssd, a, chunk=32)[0] == 5
    assert _call_scan(ssd, a, chunk=100)[0] == 5
    assert _call_scan(ssd, a, chunk=131072)[0] == 5
    assert _call_scan(ssd, a, algo=7)[0] == 5


def test_scan_rejects_aliasing(ssd):
    a = _scan_args()
    a["out"] = a["x"]
    assert _call_scan(ssd, a)[0] == 6
    a = _scan_args()
    big = torch.zeros(2 * 100 * 4 * 16, dtype=torch.bfloat16)
    a["x"] = big[: 100 * 4 * 16].view(1, 100, 4, 16)
    a["out"] = big[512: 512 + 100 * 4 * 16].view(1, 100, 4, 16)  # partial overlap
    assert _call_scan(ssd, a)[0] == 6
    a = _scan_args()
    a["final_state"] = torch.zeros(4, 16, 32)  # wrong rank
    assert _call_scan(ssd, a)[0] == 2
    a = _scan_args()
    st = torch.zeros(2, 4, 16, 32)
    a["init_state"] = st[0:1]
    a["final_state"] = st.view(-1)[16:16 + 4 * 16 * 32].view(1, 4, 16, 32)  # partial overlap
    assert _call_scan(ssd, a)[0] == 6


def _step_args(b=2, H=4, P=8, G=2, N=32, dtype=torch.bfloat16):
    return dict(state=torch.zeros(b, H, P, N), x=torch.zeros(b, H, P, dtype=dtype),
                dt=torch.zeros(b, H), A=torch.zeros(H), B=torch.zeros(b, G, N, dtype=dtype),
                C=torch.zeros(b, G, N, dtype=dtype), D=torch.zeros(H),
                out=torch.zeros(b, H, P, dtype=dtype))


STEP_CASES = [
    ("state_none", lambda a: a.update(state=None), 1),
    ("G_not_divisor", lambda a: a.update(B=torch.zeros(2, 3, 32, dtype=torch.bfloat16),
                                         C=torch.zeros(2, 3, 32, dtype=torch.bfloat16)), 2),
    ("N_unsupported", lambda a: a.update(state=torch.zeros(2, 4, 8, 24)), 5),
    ("dt_bf16", lambda a: a.update(dt=torch.zeros(2, 4, dtype=torch.bfloat16)), 3),
    ("out_aliases_x", lambda a: a.update(out=a["x"]), 6),
    ("state_noncontiguous", lambda a: a.update(state=torch.zeros(2, 4, 32, 8).transpose(2, 3)), 4),
]


@pytest.mark.parametrize("name,mutate,status", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_step_rejects(ssd, name, mutate, status):
    a = _step_args()
    mutate(a)
    lib, d = ssd.lib(), ssd.describe
    st = lib.ssd_step(d(a["state"]), d(a["x"]), d(a["dt"]), d(a["A"]), d(a["B"]), d(a["C"]),
                      d(a["D"]), d(a["out"]), None)
    assert st == status, (st, ssd.ssd_last_error())


def test_python_binding_raises(ssd):
    a = _scan_args()
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_scan_fwd(a["x"], a["dt"], a["dt_bias"], a["A"], a["B"], a["C"], a["D"],
                         a["init_state"], out=a["x"], chunk=64)
    assert e.value.status == 6


def test_host_memory_refused(ssd):
    # valid shapes in (pageable) host memory: refused before any launch,
    # whether or not a device is present
    a = _scan_args()
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_scan_fwd(a["x"], a["dt"], a["dt_bias"], a["A"], a["B"], a["C"], a["D"],
                         a["init_state"], out=a["out"], final_state=a["final_state"], chunk=64)
    assert e.value.status == 4
    b, H, P, G, N = 2, 4, 16, 2, 32
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_step(torch.zeros(b, H, P, N), torch.zeros(b, H, P, dtype=torch.bfloat16),
                     torch.zeros(b, H), -torch.ones(H), torch.zeros(b, G, N, dtype=torch.bfloat16),
                     torch.zeros(b, G, N, dtype=torch.bfloat16), torch.zeros(H),
                     out=torch.zeros(b, H, P, dtype=torch.bfloat16))
    assert e.value.status == 4


def test_plan(ssd):
    """The automatic plan, against plan timings measured on MI355X: the
    row-sliced walk for bf16 shapes whose rows fill the compute units,
    segments when the rows or (batch, head) walks are few for the sequence
    length (also for the 2.7B shape in fp32: 1024-token segments 0.92 ms,
    one walk per head 1.07 ms); always a valid segment length."""
    lib = ssd.lib()
    import ctypes as ct
    algo, seg = ct.c_int(), ct.c_int()

    def plan(b, L, H, P=64, G=1, N=128, dtype=1, cus=256):
        st = lib.ssd_scan_plan(b, L, H, P, G, N, dtype, cus, ct.byref(algo), ct.byref(seg))
        assert st == 0
        return algo.value, seg.value
    # short sequences whose (batch, head, 64-token block) workgroups fit one
    # pass over the units: the quadratic path (the tiny fp32 workload: 12.0
    # us kernel time against 19.6 us for one walk per head)
    assert plan(1, 256, 4, P=16, N=16, dtype=0) == (ssd.SSD_ALGO_QUAD, 256)
    assert plan(1, 200, 16, dtype=1) == (ssd.SSD_ALGO_QUAD, 200)
    assert plan(1, 64, 4, dtype=0)[0] != ssd.SSD_ALGO_QUAD     # one block: no chain to avoid
    assert plan(8, 256, 32)[0] != ssd.SSD_ALGO_QUAD           # 1024 workgroups: 33.5 against 18.6 us
    assert plan(1, 257, 4, dtype=0)[0] != ssd.SSD_ALGO_QUAD   # above 256 tokens
    assert plan(8, 2048, 32) == (ssd.SSD_ALGO_ROWS, 2048)    # 370M layer
    assert plan(4, 4096, 80) == (ssd.SSD_ALGO_ROWS, 4096)    # 2.7B layer
    assert plan(4, 4096, 80, dtype=0) == (ssd.SSD_ALGO_CHUNKED, 1024)
    assert plan(4, 4096, 80, N=16)[0] != ssd.SSD_ALGO_ROWS    # N=16: no row walk
    # few rows for the length: 4096-token segments measured fastest (0.39 ms
    # against 0.41 ms at 2048 and 0.53 ms at 8192)
    assert plan(1, 65536, 32, G=8) == (ssd.SSD_ALGO_CHUNKED, 4096)
    assert plan(1, 8192, 80) == (ssd.SSD_ALGO_CHUNKED, 512)   # rows 0.21 ms, 512-token segments 0.16 ms
    a, s = plan(1, 4096, 16, dtype=0)                 # 16 walks on 256 units
    assert a == ssd.SSD_ALGO_CHUNKED
    a, s = plan(1, 100, 2)
    assert a == ssd.SSD_ALGO_QUAD and s == 100
    assert lib.ssd_scan_plan(0, 10, 2, 64, 1, 128, 1, 256, ct.byref(algo), ct.byref(seg)) == 2
    assert lib.ssd_scan_plan(1, 10, 2, 64, 1, 128, 7, 256, ct.byref(algo), ct.byref(seg)) == 3


def test_rows_rejections(ssd):
    """The explicit row-sliced walk validates like the scan and rejects fp32,
    N outside {32, 64, 128} and wave counts outside 0..8."""
    lib = ssd.lib()
    d = ssd.describe

    def call(a, waves):
        return lib.ssd_scan_fwd_rows(d(a["x"]), d(a["dt"]), d(a["dt_bias"]), d(a["A"]), d(a["B"]),
                                     d(a["C"]), d(a["D"]), d(a["init_state"]), d(a["out"]),
                                     d(a["final_state"]), waves, None)
    assert call(_scan_args(dtype=torch.float32), 1) == 5
    assert call(_scan_args(N=16), 1) == 5
    assert call(_scan_args(), 9) == 5
    assert call(_scan_args(), -1) == 5
    a = _scan_args()
    a["x"] = torch.zeros(1, 99, 4, 16, dtype=torch.bfloat16)   # L disagrees with dt
    assert call(a, 1) == 2
    assert _call_scan(ssd, _scan_args(dtype=torch.float32), algo=3)[0] == 5
    assert _call_scan(ssd, _scan_args(), algo=5)[0] == 5


def test_quad_rejections(ssd):
    """The quadratic path (SSD_ALGO_QUAD) takes L <= 256 only and, for fp32
    inputs, P <= 64 (fp32 P = 128 is refused by every algorithm); the check
    comes before any device call."""
    st, msg = _call_scan(ssd, _scan_args(L=257), algo=4)
    assert st == 5 and "quadratic" in msg, (st, msg)
    st, msg = _call_scan(ssd, _scan_args(L=257, dtype=torch.float32), algo=4)
    assert st == 5 and "quadratic" in msg, (st, msg)
    # L = 256 passes the quadratic-path check and stops at the device check
    # (no GPU here; host memory on a GPU machine)
    st, msg = _call_scan(ssd, _scan_args(L=256), algo=4)
    assert st == 4 and "quadratic" not in msg, (st, msg)


def test_gated_rejections(ssd):
    """The gated scan validates like the scan, and z: present, the shape and
    element type of x, dense, not overlapping out."""
    lib, d = ssd.lib(), ssd.describe

    def call(a, z, algo=0):
        return lib.ssd_scan_fwd_gated(d(a["x"]), d(a["dt"]), d(a["dt_bias"]), d(a["A"]), d(a["B"]),
                                      d(a["C"]), d(a["D"]), d(z), d(a["init_state"]), d(a["out"]),
                                      d(a["final_state"]), 64, algo, None)
    a = _scan_args()
    assert call(a, None) == 1
    assert call(a, torch.zeros(1, 99, 4, 16, dtype=torch.bfloat16)) == 2
    assert call(a, torch.zeros(1, 100, 4, 16)) == 3
    assert call(a, torch.zeros(1, 4, 100, 16, dtype=torch.bfloat16).transpose(1, 2)) == 4
    assert call(a, a["out"]) == 6
    assert call(a, torch.zeros(1, 100, 4, 16, dtype=torch.bfloat16), algo=5) == 5
    b = _scan_args()
    b["x"] = None
    assert call(b, torch.zeros(1, 100, 4, 16, dtype=torch.bfloat16)) == 1


def _sscan_args(b=1, L=50, Dc=128, G=1, N=16, dtype=torch.bfloat16):
    return dict(x=torch.zeros(b, L, Dc, dtype=dtype), dt=torch.zeros(b, L, Dc),
                dt_bias=torch.zeros(Dc), A=-torch.ones(Dc, N), B=torch.zeros(b, L, G, N, dtype=dtype),
                C=torch.zeros(b, L, G, N, dtype=dtype), D=torch.zeros(Dc),
                init_state=torch.zeros(b, Dc, N), out=torch.zeros(b, L, Dc, dtype=dtype),
                final_state=torch.zeros(b, Dc, N))


SSCAN_CASES = [
    ("x_none", lambda a: a.update(x=None), 1),
    ("A_none", lambda a: a.update(A=None), 1),
    ("C_none", lambda a: a.update(C=None), 1),
    ("out_none", lambda a: a.update(out=None), 1),
    ("L_zero", lambda a: a.update(x=torch.zeros(1, 0, 128, dtype=torch.bfloat16)), 2),
    ("x_rank4", lambda a: a.update(x=torch.zeros(1, 50, 2, 64, dtype=torch.bfloat16)), 2),
    ("A_wrong_shape", lambda a: a.update(A=-torch.ones(16, 128)), 2),
    ("dt_wrong_shape", lambda a: a.update(dt=torch.zeros(1, 49, 128)), 2),
    ("D_not_multiple_of_G", lambda a: a.update(B=torch.zeros(1, 50, 3, 16, dtype=torch.bfloat16),
                                               C=torch.zeros(1, 50, 3, 16, dtype=torch.bfloat16)), 2),
    ("dt_bf16", lambda a: a.update(dt=torch.zeros(1, 50, 128, dtype=torch.bfloat16)), 3),
    ("B_f32_with_bf16_x", lambda a: a.update(B=torch.zeros(1, 50, 1, 16)), 3),
    ("x_noncontiguous", lambda a: a.update(
        x=torch.zeros(1, 128, 50, dtype=torch.bfloat16).transpose(1, 2)), 4),
    ("channels_per_group_not_64k", lambda a: a.update(
        x=torch.zeros(1, 50, 96, dtype=torch.bfloat16), dt=torch.zeros(1, 50, 96), dt_bias=torch.zeros(96),
        A=-torch.ones(96, 16), D=torch.zeros(96), init_state=torch.zeros(1, 96, 16),
        out=torch.zeros(1, 50, 96, dtype=torch.bfloat16), final_state=torch.zeros(1, 96, 16)), 5),
    ("N_unsupported", lambda a: a.update(A=-torch.ones(128, 32), B=torch.zeros(1, 50, 1, 32, dtype=torch.bfloat16),
                                         C=torch.zeros(1, 50, 1, 32, dtype=torch.bfloat16),
                                         init_state=torch.zeros(1, 128, 32), final_state=torch.zeros(1, 128, 32)), 5),
    ("out_aliases_x", lambda a: a.update(out=a["x"]), 6),
    ("final_overlaps_A", lambda a: a.update(final_state=a["A"].view(1, 128, 16)), 6),
]


@pytest.mark.parametrize("name,mutate,status", SSCAN_CASES, ids=[c[0] for c in SSCAN_CASES])
def test_selective_scan_rejects(ssd, name, mutate, status):
    a = _sscan_args()
    mutate(a)
    d = ssd.describe
    st = ssd.lib().ssd_selective_scan_fwd(d(a["x"]), d(a["dt"]), d(a["dt_bias"]), d(a["A"]), d(a["B"]),
                                          d(a["C"]), d(a["D"]), d(a["init_state"]), d(a["out"]),
                                          d(a["final_state"]), 0, None)
    assert st == status, (st, ssd.ssd_last_error())
    assert ssd.ssd_last_error()


def test_selective_scan_host_memory_and_segments(ssd):
    a = _sscan_args()
    d = ssd.describe
    args = [d(a[k]) for k in ("x", "dt", "dt_bias", "A", "B", "C", "D", "init_state", "out", "final_state")]
    assert ssd.lib().ssd_selective_scan_fwd(*args, -1, None) == 5      # negative segment count
    st = ssd.lib().ssd_selective_scan_fwd(*args, 0, None)               # host memory: refused
    assert st == 4, ssd.ssd_last_error()
    # final state in place of the initial state passes validation (then the
    # host memory is refused)
    a["final_state"] = a["init_state"]
    args = [d(a[k]) for k in ("x", "dt", "dt_bias", "A", "B", "C", "D", "init_state", "out", "final_state")]
    assert ssd.lib().ssd_selective_scan_fwd(*args, 0, None) == 4


def test_selective_scan_oversized(ssd):
    # one 2^24-token sequence of 65536 channels: even 1024 segments leave a
    # segment above the 32-bit byte range; refused on the host
    b, L, Dc, G, N = 1, 1 << 24, 1 << 16, 1, 16
    bf, f32 = 1, 0
    ts = [_fake(ssd, (b, L, Dc), bf, 1), _fake(ssd, (b, L, Dc), f32, 2), None,
          _fake(ssd, (Dc, N), f32, 3), _fake(ssd, (b, L, G, N), bf, 4), _fake(ssd, (b, L, G, N), bf, 5),
          None, None, _fake(ssd, (b, L, Dc), bf, 6), None]
    ptrs = [ctypes.byref(t) if t is not None else None for t in ts]
    st = ssd.lib().ssd_selective_scan_fwd(*ptrs, 0, None)
    assert st == 5, (st, ssd.ssd_last_error())
    assert "too large" in ssd.ssd_last_error()


def test_last_error_is_per_thread(ssd):
    # each thread sees the message of its own last call
    import threading
    msgs, errs = {}, []

    def worker(i):
        try:
            for _ in range(50):
                a = _scan_args()
                if i % 2:
                    a["x"] = None
                    st, msg = _call_scan(ssd, a)
                    assert st == 1 and "x" in msg, msg
                else:
                    st, msg = _call_scan(ssd, a, chunk=32)
                    assert st == 5 and "chunk" in msg, msg
            msgs[i] = msg
        except AssertionError as e:
            errs.append(str(e))
    ts = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errs, errs[:3]
    assert len(msgs) == 8


# --- gradients (ssd_scan_bwd): host-side validation, no device call -------

def _bwd_args(b=1, L=100, H=4, P=32, G=2, N=32, dtype=torch.bfloat16):
    a = _scan_args(b, L, H, P, G, N, dtype)
    del a["out"], a["final_state"]
    a.update(dout=torch.zeros(b, L, H, P, dtype=dtype), dfinal_state=torch.zeros(b, H, P, N),
             dx=torch.zeros(b, L, H, P), ddt=torch.zeros(b, L, H), ddt_bias=torch.zeros(H),
             dA=torch.zeros(H), dB=torch.zeros(b, L, G, N), dC=torch.zeros(b, L, G, N),
             dD=torch.zeros(H), dinit_state=torch.zeros(b, H, P, N))
    return a


BWD_ORDER = ["x", "dt", "dt_bias", "A", "B", "C", "D", "init_state", "dout", "dfinal_state",
             "dx", "ddt", "ddt_bias", "dA", "dB", "dC", "dD", "dinit_state"]


def _call_bwd(ssd, a):
    d = ssd.describe
    st = ssd.lib().ssd_scan_bwd(*[d(a[k]) for k in BWD_ORDER], None)
    return st, ssd.ssd_last_error()


BWD_CASES = [
    ("dout_none", lambda a: a.update(dout=None), 1),
    ("dx_none", lambda a: a.update(dx=None), 1),
    ("dA_none", lambda a: a.update(dA=None), 1),
    ("dB_none", lambda a: a.update(dB=None), 1),
    ("ddt_none", lambda a: a.update(ddt=None), 1),
    ("dout_dtype", lambda a: a.update(dout=torch.zeros(1, 100, 4, 32)), 3),
    ("dx_bf16", lambda a: a.update(dx=torch.zeros(1, 100, 4, 32, dtype=torch.bfloat16)), 3),
    ("dC_shape", lambda a: a.update(dC=torch.zeros(1, 100, 2, 16)), 2),
    ("ddt_shape", lambda a: a.update(ddt=torch.zeros(1, 100, 3)), 2),
    ("dinit_shape", lambda a: a.update(dinit_state=torch.zeros(1, 4, 32, 16)), 2),
    ("dfinal_shape", lambda a: a.update(dfinal_state=torch.zeros(1, 4, 16, 32)), 2),
    ("dx_strided", lambda a: a.update(dx=torch.zeros(1, 100, 4, 64)[..., ::2]), 4),
    ("dx_aliases_x", lambda a: a.update(dx=a["x"]), 3),
    ("dB_aliases_dC", lambda a: a.update(dB=a["dC"]), 6),
    ("ddt_aliases_dt", lambda a: a.update(ddt=a["dt"]), 6),
    ("dinit_aliases_init", lambda a: a.update(dinit_state=a["init_state"]), 6),
]


@pytest.mark.parametrize("name,mutate,status", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_bwd_rejects(ssd, name, mutate, status):
    a = _bwd_args()
    mutate(a)
    st, msg = _call_bwd(ssd, a)
    assert st == status, (st, msg)
    assert msg


@pytest.mark.parametrize("P,N", [(128, 32), (128, 128)])
def test_bwd_rejects_unsupported_sizes(ssd, P, N):
    # P = 128 (bf16 forward only) is not supported by the backward
    a = _bwd_args(P=P, N=N)
    st, msg = _call_bwd(ssd, a)
    assert st == 5 and "backward" in msg, (st, msg)


def test_bwd_host_memory_refused(ssd):
    # valid shapes in pageable host memory: refused before any launch
    # (with no device present the refusal names the missing device instead)
    st, msg = _call_bwd(ssd, _bwd_args())
    assert st == 4 and msg, (st, msg)


GATED_ORDER = ["x", "dt", "dt_bias", "A", "B", "C", "D", "z", "init_state", "dout", "dfinal_state",
               "dx", "ddt", "ddt_bias", "dA", "dB", "dC", "dD", "dz", "dinit_state"]


def _gated_bwd_args():
    a = _bwd_args()
    a.update(z=torch.zeros(1, 100, 4, 32, dtype=torch.bfloat16), dz=torch.zeros(1, 100, 4, 32))
    return a


def _call_gated_bwd(ssd, a):
    d = ssd.describe
    st = ssd.lib().ssd_scan_bwd_gated(*[d(a[k]) for k in GATED_ORDER], None)
    return st, ssd.ssd_last_error()


GATED_BWD_CASES = [
    ("z_none", lambda a: a.update(z=None), 1),
    ("dz_none", lambda a: a.update(dz=None), 1),
    ("z_dtype", lambda a: a.update(z=torch.zeros(1, 100, 4, 32)), 3),
    ("dz_bf16", lambda a: a.update(dz=torch.zeros(1, 100, 4, 32, dtype=torch.bfloat16)), 3),
    ("dz_shape", lambda a: a.update(dz=torch.zeros(1, 100, 4, 16)), 2),
    ("dz_aliases_dx", lambda a: a.update(dz=a["dx"]), 6),
    ("dx_aliases_z_storage", lambda a: a.update(dx=torch.zeros(1, 100, 4, 32), z=None), 1),
]


@pytest.mark.parametrize("name,mutate,status", GATED_BWD_CASES, ids=[c[0] for c in GATED_BWD_CASES])
def test_gated_bwd_rejects(ssd, name, mutate, status):
    a = _gated_bwd_args()
    mutate(a)
    st, msg = _call_gated_bwd(ssd, a)
    assert st == status, (st, msg)
    assert msg


def test_gated_bwd_output_overlapping_z(ssd):
    a = _gated_bwd_args()
    buf = torch.zeros(2 * 100 * 4 * 32)
    a["dz"] = buf[: 100 * 4 * 32].view(1, 100, 4, 32)
    a["z"] = torch.zeros(1, 100, 4, 32, dtype=torch.bfloat16)
    a["dx"] = buf[100 * 4 * 32 - 64: 2 * 100 * 4 * 32 - 64].view(1, 100, 4, 32)  # overlaps dz
    assert _call_gated_bwd(ssd, a)[0] == 6
