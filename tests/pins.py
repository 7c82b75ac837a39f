"""Independent checks that pin the fp64 oracle to the pages and to mathematics.

Each ``pin_*`` function takes an oracle object (``scan``/``step`` methods)
and raises ``AssertionError`` when the oracle disagrees with a result that is
fixed independently of the oracle's own loop:

* ``pin_golden``      hand-worked examples (tests/golden/hand_examples.txt)
* ``pin_quadratic``   brute-force matrix form Y = (L o C B^T) diag(Delta) X
                      with the mask built as products of forget gates
                      ("Mamba-3 deep dive ch. 2", section 2.2.1), plus the
                      initial-state and D terms, and the final state
* ``pin_no_decay``    A = 0 closed form: prefix sums of Delta x B^T
* ``pin_scalar_state`` N = 1: scalar-decay linear attention
                      (same page, section 2.2.2)
* ``pin_split``       carried state: two half-scans equal one scan
* ``pin_lti``         constant parameters: convolution with numpy.convolve
                      (Mamba reading notes, LTI section; "Transformers are
                      SSMs" summary, section 1.1)
* ``pin_step_scan``   T single steps equal one T-token scan
* ``pin_exact_int``   integer data with A = 0, Delta = 1: exact integers
* ``pin_linearity``, ``pin_groups``, ``pin_head_perm``, ``pin_decay_bound``
* ``pin_gate_closed_forms`` the output gate y * silu(z) at z = 0, +-ln 3
                      (logistic 3/4 and 1/4) and +-40
* ``pin_gate_expit``  the gate against ``scipy.special.expit`` (a library
                      logistic)
* ``pin_sscan_closed_form`` the selective scan with a diagonal A per
                      (channel, n): per state index an explicit double sum
                      of decays exp(A (S_t - S_s)), S the cumulative sum of
                      Delta (Mamba reading notes, selective mechanism)
* ``pin_sscan_reduces_to_ssd`` A constant over n: the selective scan equals
                      the (separately pinned) SSD scan with one channel per
                      head
* ``pin_sscan_hand``  a hand-worked 3-token example with two state indices
* ``pin_bwd_finite_difference`` every gradient of the scan against central
                      differences of the forward scan along random directions
* ``pin_bwd_transpose`` dx, dinit, dD exactly as transposes of the explicit
                      L x L operator (the forward is linear in x and h0)
* ``pin_bwd_hand``    a one-token gradient example worked by hand
* ``pin_bwd_gated_finite_difference`` gradients of the gated scan (and dz)
                      against central differences of the gated forward

Softplus here is ``numpy.logaddexp(0, z)`` (a library routine).
"""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "hand_examples.txt")


def softplus(z):
    return np.logaddexp(0.0, z)


def rand_case(rng, b, L, H, P, G, N, *, A_scale=1.0, init=True, dt_shift=-1.0):
    """Generic float64 inputs for oracle self-checks."""
    x = rng.standard_normal((b, L, H, P))
    dt = 0.5 * rng.standard_normal((b, L, H))
    dt_bias = dt_shift + 0.3 * rng.standard_normal(H)
    A = -A_scale * np.exp(rng.uniform(0.0, np.log(4.0), H))
    B = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    C = rng.standard_normal((b, L, G, N)) / np.sqrt(N)
    D = rng.standard_normal(H)
    h0 = 0.5 * rng.standard_normal((b, H, P, N)) if init else None
    return dict(x=x, dt=dt, dt_bias=dt_bias, A=A, B=B, C=C, D=D, init=h0)


def _close(a, b, rtol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b))) if a.size else 0.0
    assert err <= rtol, "%s: max rel err %.3e > %.1e" % (what, err, rtol)


# --------------------------------------------------------------------------
def read_golden(path=GOLDEN):
    cases, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0]}
            cases.append(cur)
        else:
            cur[key] = np.array([float(v) for v in vals])
    out = []
    for c in cases:
        b, L, H, P, G, N = (int(v) for v in c["dims"])
        out.append(dict(
            name=c["name"], x=c["x"].reshape(b, L, H, P), dt=c["dt"].reshape(b, L, H),
            dt_bias=c["dt_bias"].reshape(H), A=c["A"].reshape(H),
            B=c["B"].reshape(b, L, G, N), C=c["C"].reshape(b, L, G, N),
            D=c["D"].reshape(H),
            init=c["init"].reshape(b, H, P, N) if "init" in c else None,
            y=c["y"].reshape(b, L, H, P), final=c["final"].reshape(b, H, P, N)))
    return out


def pin_golden(o):
    for c in read_golden():
        y, fin = o.scan(c["x"], c["dt"], c["dt_bias"], c["A"], c["B"], c["C"],
                        c["D"], c["init"])
        _close(y, c["y"], 1e-12, "golden %s y" % c["name"])
        _close(fin, c["final"], 1e-12, "golden %s final" % c["name"])


# --------------------------------------------------------------------------
def quadratic_form(x, dt, dt_bias, A, B, C, D, init):
    """Brute-force matrix form, O(L^2) per (batch, head)."""
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    delta = softplus(dt + dt_bias[None, None, :])
    alpha = np.exp(delta * A[None, None, :])
    y = np.zeros((b, L, H, P))
    fin = np.zeros((b, H, P, N))
    for ib in range(b):
        for h in range(H):
            g = h * G // H
            Bm, Cm = B[ib, :, g, :], C[ib, :, g, :]
            al, de, X = alpha[ib, :, h], delta[ib, :, h], x[ib, :, h, :]
            mask = np.zeros((L, L))
            for i in range(L):
                mask[i, i] = 1.0
                for j in range(i - 1, -1, -1):
                    mask[i, j] = mask[i, j + 1] * al[j + 1]
            M = mask * (Cm @ Bm.T) * de[None, :]
            Y = M @ X + D[h] * X
            carry = np.array([np.prod(al[s + 1:]) for s in range(L)]) * de
            F = (X * carry[:, None]).T @ Bm
            if init is not None:
                dec = np.array([np.prod(al[: i + 1]) for i in range(L)])
                Y = Y + dec[:, None] * (Cm @ init[ib, h].T)
                F = F + np.prod(al) * init[ib, h]
            y[ib, :, h, :] = Y
            fin[ib, h] = F
    return y, fin


def pin_quadratic(o, seed=11):
    rng = np.random.default_rng(seed)
    for (b, L, H, P, G, N) in [(1, 64, 2, 3, 1, 5), (2, 17, 4, 2, 2, 3), (1, 40, 3, 4, 3, 1)]:
        c = rand_case(rng, b, L, H, P, G, N)
        y, fin = o.scan(**c)
        yq, fq = quadratic_form(**c)
        _close(y, yq, 1e-12, "quadratic y %s" % ((b, L, H, P, G, N),))
        _close(fin, fq, 1e-12, "quadratic final")


def pin_no_decay(o, seed=12):
    rng = np.random.default_rng(seed)
    b, L, H, P, G, N = 2, 50, 2, 3, 1, 4
    c = rand_case(rng, b, L, H, P, G, N)
    c["A"] = np.zeros(H)
    y, fin = o.scan(**c)
    delta = softplus(c["dt"] + c["dt_bias"])
    for ib in range(b):
        for h in range(H):
            Bm, Cm = c["B"][ib, :, 0, :], c["C"][ib, :, 0, :]
            X = c["x"][ib, :, h, :]
            outer = (delta[ib, :, h][:, None, None] * X[:, :, None]) * Bm[:, None, :]
            Hs = c["init"][ib, h][None] + np.cumsum(outer, axis=0)     # [L,P,N]
            Y = np.einsum("tpn,tn->tp", Hs, Cm) + c["D"][h] * X
            _close(y[ib, :, h, :], Y, 1e-12, "A=0 y")
            _close(fin[ib, h], Hs[-1], 1e-12, "A=0 final")


def pin_scalar_state(o, seed=13):
    rng = np.random.default_rng(seed)
    b, L, H, P, G, N = 1, 48, 3, 4, 1, 1
    c = rand_case(rng, b, L, H, P, G, N)
    y, fin = o.scan(**c)
    delta = softplus(c["dt"] + c["dt_bias"])
    for h in range(H):
        cum = np.cumsum(delta[0, :, h] * c["A"][h])      # log of the running decay
        bb, cc = c["B"][0, :, 0, 0], c["C"][0, :, 0, 0]
        X = c["x"][0, :, h, :]
        q = cc * np.exp(cum)                            # query side
        k = bb * np.exp(-cum) * delta[0, :, h]          # key side
        Y = q[:, None] * np.cumsum(k[:, None] * X, axis=0)
        Y += q[:, None] * c["init"][0, h][:, 0][None, :] + c["D"][h] * X
        _close(y[0, :, h, :], Y, 1e-11, "N=1 linear attention")
        F = np.exp(cum[-1]) * (np.sum(k[:, None] * X, axis=0) + c["init"][0, h][:, 0])
        _close(fin[0, h, :, 0], F, 1e-11, "N=1 final")


def pin_split(o, seed=14):
    rng = np.random.default_rng(seed)
    b, L, H, P, G, N = 2, 70, 4, 3, 2, 5
    c = rand_case(rng, b, L, H, P, G, N)
    y, fin = o.scan(**c)
    for L1 in (1, 33, 69):
        a = {k: v for k, v in c.items()}
        a.update(x=c["x"][:, :L1], dt=c["dt"][:, :L1], B=c["B"][:, :L1], C=c["C"][:, :L1])
        y1, h1 = o.scan(**a)
        a.update(x=c["x"][:, L1:], dt=c["dt"][:, L1:], B=c["B"][:, L1:], C=c["C"][:, L1:],
                 init=h1)
        y2, h2 = o.scan(**a)
        _close(np.concatenate([y1, y2], axis=1), y, 1e-12, "split y L1=%d" % L1)
        _close(h2, fin, 1e-12, "split final L1=%d" % L1)


def pin_lti(o, seed=15):
    rng = np.random.default_rng(seed)
    b, L, H, P, G, N = 1, 60, 2, 3, 1, 4
    c = rand_case(rng, b, L, H, P, G, N, init=False)
    c["dt"] = np.broadcast_to(c["dt"][:, :1, :], (b, L, H)).copy()
    c["B"] = np.broadcast_to(c["B"][:, :1], (b, L, G, N)).copy()
    c["C"] = np.broadcast_to(c["C"][:, :1], (b, L, G, N)).copy()
    y, _ = o.scan(**c)
    for h in range(H):
        de = softplus(c["dt"][0, 0, h] + c["dt_bias"][h])
        al = np.exp(de * c["A"][h])
        cb = float(c["C"][0, 0, 0] @ c["B"][0, 0, 0])
        kern = de * cb * al ** np.arange(L)
        for p in range(P):
            X = c["x"][0, :, h, p]
            Y = np.convolve(kern, X)[:L] + c["D"][h] * X
            _close(y[0, :, h, p], Y, 1e-12, "LTI convolution")


def pin_step_scan(o, seed=16):
    rng = np.random.default_rng(seed)
    b, L, H, P, G, N = 2, 20, 4, 3, 2, 5
    c = rand_case(rng, b, L, H, P, G, N)
    y, fin = o.scan(**c)
    delta = softplus(c["dt"] + c["dt_bias"][None, None, :])
    S = c["init"]
    for t in range(L):
        yt, S = o.step(S, c["x"][:, t], delta[:, t], c["A"], c["B"][:, t], c["C"][:, t], c["D"])
        _close(yt, y[:, t], 1e-12, "step vs scan y t=%d" % t)
    _close(S, fin, 1e-12, "step vs scan final")


def pin_exact_int(o, seed=17):
    """A = 0, Delta = 1, small integers: every value is an exact integer."""
    rng = np.random.default_rng(seed)
    b, H, P, G, N, T = 2, 4, 3, 2, 6, 5
    S = rng.integers(-3, 4, (b, H, P, N)).astype(np.int64)
    A = np.zeros(H)
    D = rng.integers(-2, 3, H).astype(np.int64)
    S_f = S.astype(np.float64)
    for _ in range(T):
        x = rng.integers(-4, 5, (b, H, P))
        Bm = rng.integers(-3, 4, (b, G, N))
        Cm = rng.integers(-3, 4, (b, G, N))
        y, S_f = o.step(S_f, x, np.ones((b, H)), A, Bm, Cm, D)
        g = np.arange(H) * G // H
        S = S + x[:, :, :, None] * Bm[:, g, None, :]
        y_int = np.einsum("bhpn,bhn->bhp", S, Cm[:, g, :]) + D[None, :, None] * x
        assert np.array_equal(y, y_int.astype(np.float64)), "exact integer y"
        assert np.array_equal(S_f, S.astype(np.float64)), "exact integer state"


def pin_linearity(o, seed=18):
    rng = np.random.default_rng(seed)
    c = rand_case(rng, 1, 33, 2, 3, 1, 4)
    y, fin = o.scan(**c)
    z = dict(c, init=None)
    y0, f0 = o.scan(**z)
    yh, fh = o.scan(**dict(c, x=np.zeros_like(c["x"]), D=np.zeros_like(c["D"])))
    _close(y, y0 + yh, 1e-12, "linearity in (x, h0)")
    _close(fin, f0 + fh, 1e-12, "linearity final")
    y3, f3 = o.scan(**dict(z, x=-2.5 * c["x"]))
    _close(y3, -2.5 * y0, 1e-12, "homogeneity y")
    _close(f3, -2.5 * f0, 1e-12, "homogeneity final")


def pin_groups(o, seed=19):
    rng = np.random.default_rng(seed)
    b, L, H, P, G, N = 2, 25, 6, 2, 3, 4
    c = rand_case(rng, b, L, H, P, G, N)
    y, fin = o.scan(**c)
    g = np.arange(H) * G // H
    r = dict(c, B=c["B"][:, :, g, :], C=c["C"][:, :, g, :])
    yr, fr = o.scan(**r)
    _close(y, yr, 0.0, "groups vs repeated")
    _close(fin, fr, 0.0, "groups vs repeated final")
    one = dict(c, B=np.repeat(c["B"][:, :, :1], G, 2), C=np.repeat(c["C"][:, :, :1], G, 2))
    y1, _ = o.scan(**one)
    y2, _ = o.scan(**dict(c, B=c["B"][:, :, :1], C=c["C"][:, :, :1]))
    _close(y1, y2, 0.0, "equal groups vs G=1")


def pin_head_perm(o, seed=20):
    rng = np.random.default_rng(seed)
    b, L, H, P, G, N = 1, 21, 5, 2, 1, 3
    c = rand_case(rng, b, L, H, P, G, N)
    y, fin = o.scan(**c)
    perm = rng.permutation(H)
    pc = dict(c, x=c["x"][:, :, perm], dt=c["dt"][:, :, perm], dt_bias=c["dt_bias"][perm],
              A=c["A"][perm], D=c["D"][perm], init=c["init"][:, perm])
    yp, fp = o.scan(**pc)
    _close(yp, y[:, :, perm], 0.0, "head permutation")
    _close(fp, fin[:, perm], 0.0, "head permutation final")


def pin_decay_bound(o, seed=21):
    rng = np.random.default_rng(seed)
    c = rand_case(rng, 1, 30, 3, 2, 1, 4)
    c["x"] = np.zeros_like(c["x"])
    prev = np.abs(c["init"]).copy()
    S = c["init"]
    delta = softplus(c["dt"] + c["dt_bias"])
    for t in range(30):
        _, S = o.step(S, c["x"][:, t], delta[:, t], c["A"], c["B"][:, t], c["C"][:, t], c["D"])
        assert np.all(np.abs(S) <= prev + 1e-15), "state grew with zero input"
        assert np.all(np.abs(S) < prev + 1e-15) or np.all(prev == 0)
        prev = np.abs(S)


def pin_gate_closed_forms(o):
    # silu(v) = v * logistic(v); logistic(ln 3) = 3/4, logistic(-ln 3) = 1/4,
    # logistic(0) = 1/2 (so silu(0) = 0 exactly); for v = 40 the logistic is 1
    # to double precision, for v = -40 it is e^v / (1 + e^v)
    l3 = np.log(3.0)
    y = np.array([2.5, -1.5, 3.0, 0.7, -2.0, 1.25])
    z = np.array([0.0, 0.0, l3, -l3, 40.0, -40.0])
    want = np.array([0.0, 0.0, 3.0 * 0.75 * l3, 0.7 * 0.25 * -l3, -2.0 * 40.0,
                     1.25 * -40.0 * np.exp(-40.0) / (1.0 + np.exp(-40.0))])
    got = o.gate(y, z)
    assert got[0] == 0.0 and got[1] == 0.0, "silu(0) must be exactly 0"
    _close(got, want, 1e-15, "gate closed forms")
    assert abs(got[5] - want[5]) <= 1e-15 * abs(want[5]), "gate far negative tail"


def pin_gate_expit(o, seed=22):
    from scipy.special import expit
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((3, 17, 5))
    z = 4.0 * rng.standard_normal((3, 17, 5))
    _close(o.gate(y, z), y * z * expit(z), 1e-15, "gate vs scipy expit")


def rand_sscan_case(rng, b, L, Dc, G, N):
    """Generic float64 inputs for the selective scan (A distinct per
    (channel, n))."""
    return dict(x=rng.standard_normal((b, L, Dc)), dt=0.5 * rng.standard_normal((b, L, Dc)),
                dt_bias=-1.0 + 0.3 * rng.standard_normal(Dc),
                A=-np.exp(rng.uniform(np.log(0.5), np.log(4.0), (Dc, N))),
                B=rng.standard_normal((b, L, G, N)) / np.sqrt(N),
                C=rng.standard_normal((b, L, G, N)) / np.sqrt(N),
                D=rng.standard_normal(Dc), init=0.5 * rng.standard_normal((b, Dc, N)))


def sscan_closed_form(x, dt, dt_bias, A, B, C, D, init):
    """Per state index n the selective recurrence is a scalar linear
    recurrence with gate exp(A[d,n] Delta_t); unrolled,
        h_t[n] = exp(A S_t) h0[n] + sum_{s<=t} exp(A (S_t - S_s)) Delta_s B_s[n] x_s
    with S the inclusive cumulative sum of Delta.  Evaluated as an explicit
    double sum (no recurrence)."""
    b, L, Dc = x.shape
    G, N = B.shape[2], B.shape[3]
    delta = softplus(dt + dt_bias)
    S = np.cumsum(delta, axis=1)
    tri = np.tril(np.ones((L, L), dtype=bool))[:, :, None]
    y = np.empty_like(x)
    fin = np.empty((b, Dc, N))
    for ib in range(b):
        for d in range(Dc):
            g = (d * G) // Dc
            Sd = S[ib, :, d]
            arg = A[d][None, None, :] * (Sd[:, None, None] - Sd[None, :, None])
            dec = np.exp(np.where(tri, arg, -np.inf))                      # [t, s, N]
            inp = (delta[ib, :, d] * x[ib, :, d])[:, None] * B[ib, :, g, :]  # [s, N]
            Hs = np.einsum("tsn,sn->tn", dec, inp) + np.exp(A[d][None, :] * Sd[:, None]) * init[ib, d][None, :]
            y[ib, :, d] = np.einsum("tn,tn->t", Hs, C[ib, :, g, :]) + D[d] * x[ib, :, d]
            fin[ib, d] = Hs[-1]
    return y, fin


def pin_sscan_closed_form(o, seed=23):
    rng = np.random.default_rng(seed)
    for (b, L, Dc, G, N) in [(1, 40, 5, 1, 4), (2, 23, 6, 3, 3), (1, 31, 4, 2, 16)]:
        c = rand_sscan_case(rng, b, L, Dc, G, N)
        y, fin = o.selective_scan(**c)
        yq, fq = sscan_closed_form(**c)
        _close(y, yq, 1e-12, "selective scan closed form y %s" % ((b, L, Dc, G, N),))
        _close(fin, fq, 1e-12, "selective scan closed form final")


def pin_sscan_reduces_to_ssd(o, seed=24):
    # with A[d, n] = a_d for every n the selective scan is the SSD scan with
    # H = Dc heads of P = 1 channel each (same group map floor(h G / H))
    rng = np.random.default_rng(seed)
    b, L, Dc, G, N = 2, 37, 6, 2, 8
    c = rand_sscan_case(rng, b, L, Dc, G, N)
    a = -np.exp(rng.uniform(np.log(0.5), np.log(4.0), Dc))
    c["A"] = np.repeat(a[:, None], N, axis=1)
    y, fin = o.selective_scan(**c)
    ys, fs = o.scan(c["x"][..., None], c["dt"], c["dt_bias"], a, c["B"], c["C"], c["D"],
                    c["init"][:, :, None, :])
    _close(y, ys[..., 0], 1e-13, "selective scan vs SSD y")
    _close(fin, fs[:, :, 0, :], 1e-13, "selective scan vs SSD final")


def pin_sscan_hand(o):
    # One channel, N = 2, A = [-ln 2, 0], Delta = 1 (dt = ln(e - 1)), D = 0.5,
    # h0 = [4, -2], x = [1, 2, 3], B = [[1,0],[0,1],[1,1]], C = [[1,1],[1,0],[0,1]].
    # Gates exp(Delta A) = [1/2, 1]:
    #   t0: h = [2 + 1, -2 + 0] = [3, -2];      y = 3 - 2 + 0.5 = 1.5
    #   t1: h = [1.5 + 0, -2 + 2] = [1.5, 0];   y = 1.5 + 1.0  = 2.5
    #   t2: h = [0.75 + 3, 0 + 3] = [3.75, 3];  y = 3 + 1.5    = 4.5
    c = dict(x=np.array([[[1.0], [2.0], [3.0]]]), dt=np.full((1, 3, 1), np.log(np.e - 1.0)),
             dt_bias=np.zeros(1), A=np.array([[-np.log(2.0), 0.0]]),
             B=np.array([[[[1.0, 0.0]], [[0.0, 1.0]], [[1.0, 1.0]]]]),
             C=np.array([[[[1.0, 1.0]], [[1.0, 0.0]], [[0.0, 1.0]]]]),
             D=np.array([0.5]), init=np.array([[[4.0, -2.0]]]))
    y, fin = o.selective_scan(**c)
    _close(y[0, :, 0], [1.5, 2.5, 4.5], 1e-14, "selective scan hand example y")
    _close(fin[0, 0], [3.75, 3.0], 1e-14, "selective scan hand example final")


# --------------------------------------------------------------------------
# Gradients of the scan (oracle ``scan_bwd``).  Objective
# Lobj = sum <dy, y> + <dfinal, final state>.

BWD_KEYS = ["x", "dt", "dt_bias", "A", "B", "C", "D", "init"]
GRAD_OF = dict(x="dx", dt="ddt", dt_bias="ddt_bias", A="dA", B="dB", C="dC", D="dD", init="dinit")


def _objective(o, case, dy, dfinal):
    y, fin = o.scan(**case)
    return float(np.sum(dy * y) + (np.sum(dfinal * fin) if dfinal is not None else 0.0))


def pin_bwd_finite_difference(o, seed=25):
    """Every gradient against central differences of the (separately pinned)
    forward scan along a random direction: (Lobj(p + e v) - Lobj(p - e v)) / 2e
    equals <grad, v> up to O(e^2) (e = 1e-5, fp64)."""
    rng = np.random.default_rng(seed)
    for (b, L, H, P, G, N, init, fin) in [(2, 9, 4, 3, 2, 5, True, True), (1, 6, 2, 2, 1, 3, False, False)]:
        case = rand_case(rng, b, L, H, P, G, N, init=init)
        if case["init"] is None:
            case["init"] = np.zeros((b, H, P, N))
        dy = rng.standard_normal((b, L, H, P))
        dfinal = rng.standard_normal((b, H, P, N)) if fin else None
        grads = o.scan_bwd(**case, dy=dy, dfinal=dfinal)
        eps = 1e-5
        for k in BWD_KEYS:
            v = rng.standard_normal(case[k].shape)
            plus = dict(case, **{k: case[k] + eps * v})
            minus = dict(case, **{k: case[k] - eps * v})
            fd = (_objective(o, plus, dy, dfinal) - _objective(o, minus, dy, dfinal)) / (2 * eps)
            an = float(np.sum(grads[GRAD_OF[k]] * v))
            assert abs(fd - an) <= 1e-6 * (1.0 + abs(fd)), (k, fd, an)


def pin_bwd_transpose(o, seed=26):
    """dx, dinit and dD exactly: y and the final state are linear in x and in
    the initial state, so these gradients are the transposes of the explicit
    L x L operator M = mask o (C B^T) diag(Delta) (mask entries: products of
    forget gates), of the decay read-out of the initial state and of the
    final-state carry, applied to dy and dfinal."""
    rng = np.random.default_rng(seed)
    b, L, H, P, G, N = 2, 11, 4, 3, 2, 4
    c = rand_case(rng, b, L, H, P, G, N)
    dy = rng.standard_normal((b, L, H, P))
    dfinal = rng.standard_normal((b, H, P, N))
    grads = o.scan_bwd(**c, dy=dy, dfinal=dfinal)
    delta = softplus(c["dt"] + c["dt_bias"][None, None, :])
    alpha = np.exp(delta * c["A"][None, None, :])
    dx = np.zeros_like(c["x"])
    dinit = np.zeros_like(c["init"])
    dD = np.zeros(H)
    for ib in range(b):
        for h in range(H):
            g = h * G // H
            Bm, Cm = c["B"][ib, :, g, :], c["C"][ib, :, g, :]
            al, de = alpha[ib, :, h], delta[ib, :, h]
            mask = np.zeros((L, L))
            for i in range(L):
                mask[i, i] = 1.0
                for j in range(i - 1, -1, -1):
                    mask[i, j] = mask[i, j + 1] * al[j + 1]
            M = mask * (Cm @ Bm.T) * de[None, :]
            carry = np.array([np.prod(al[s + 1:]) for s in range(L)]) * de      # final state: sum_s carry_s x_s B_s^T
            dec = np.array([np.prod(al[: i + 1]) for i in range(L)])            # y_i gets dec_i * init C_i
            Y = dy[ib, :, h, :]
            dx[ib, :, h, :] = M.T @ Y + c["D"][h] * Y + carry[:, None] * (Bm @ dfinal[ib, h].T)
            dinit[ib, h] = (dec[:, None] * Y).T @ Cm + np.prod(al) * dfinal[ib, h]
            dD[h] += np.sum(Y * c["x"][ib, :, h, :])
    _close(grads["dx"], dx, 1e-12, "dx vs transposed operator")
    _close(grads["dinit"], dinit, 1e-12, "dinit vs transposed operator")
    _close(grads["dD"], dD, 1e-12, "dD")


def pin_bwd_hand(o):
    """One token, one head, P = N = 1, worked by hand.  h = alpha h0 + Delta x B,
    y = h C + D x, Lobj = dy y + df h.  With u = dy C + df (all that reaches h):
    dx = D dy + Delta B u, dB = Delta x u, dC = dy h, dD = dy x, dh0 = alpha u,
    dDelta = u (A alpha h0 + x B), dA = u Delta alpha h0, ddt = dDelta sigmoid(z).
    Values: z = ln(e - 1) (so Delta = 1), A = -ln 2 (alpha = 1/2), x = 2, B = 3,
    C = 5, D = 7, h0 = 4, dy = 1, df = 10: h = 8, u = 15, sigmoid(z) = (e-1)/e."""
    e = np.e
    case = dict(x=np.full((1, 1, 1, 1), 2.0), dt=np.full((1, 1, 1), np.log(e - 1.0)),
                dt_bias=np.zeros(1), A=np.full(1, -np.log(2.0)), B=np.full((1, 1, 1, 1), 3.0),
                C=np.full((1, 1, 1, 1), 5.0), D=np.full(1, 7.0), init=np.full((1, 1, 1, 1), 4.0))
    g = o.scan_bwd(**case, dy=np.ones((1, 1, 1, 1)), dfinal=np.full((1, 1, 1, 1), 10.0))
    d_delta = 15.0 * (-np.log(2.0) * 0.5 * 4.0 + 2.0 * 3.0)
    want = dict(dx=7.0 + 45.0, dB=30.0, dC=8.0, dD=2.0, dinit=7.5, dA=30.0,
                ddt=d_delta * (e - 1.0) / e, ddt_bias=d_delta * (e - 1.0) / e)
    for k, v in want.items():
        _close(g[k].ravel(), np.array([v]), 1e-12, "hand " + k)


def pin_bwd_gated_finite_difference(o, seed=27):
    """Gradients of the gated scan (scan_bwd_gated, with dz) against central
    differences of the (separately pinned) gated forward along random
    directions, every input and z."""
    rng = np.random.default_rng(seed)
    b, L, H, P, G, N = 2, 7, 4, 3, 2, 4
    case = rand_case(rng, b, L, H, P, G, N)
    z = 1.5 * rng.standard_normal((b, L, H, P))
    dout = rng.standard_normal((b, L, H, P))
    dfinal = rng.standard_normal((b, H, P, N))
    g = o.scan_bwd_gated(case["x"], case["dt"], case["dt_bias"], case["A"], case["B"], case["C"], z,
                         case["D"], case["init"], dout, dfinal)

    def obj(c, zz):
        y = o.gate(o.scan(**c, want_final=False)[0], zz)
        return float(np.sum(dout * y) + np.sum(dfinal * o.scan(**c)[1]))
    eps = 1e-5
    for k in BWD_KEYS + ["z"]:
        v = rng.standard_normal(z.shape if k == "z" else case[k].shape)
        if k == "z":
            fd = (obj(case, z + eps * v) - obj(case, z - eps * v)) / (2 * eps)
            an = float(np.sum(g["dz"] * v))
        else:
            fd = (obj(dict(case, **{k: case[k] + eps * v}), z) - obj(dict(case, **{k: case[k] - eps * v}), z)) / (2 * eps)
            an = float(np.sum(g[GRAD_OF[k]] * v))
        assert abs(fd - an) <= 1e-6 * (1.0 + abs(fd)), (k, fd, an)


ALL_PINS = [pin_golden, pin_quadratic, pin_no_decay, pin_scalar_state, pin_split,
            pin_lti, pin_step_scan, pin_exact_int, pin_linearity, pin_groups,
            pin_head_perm, pin_decay_bound, pin_gate_closed_forms, pin_gate_expit,
            pin_sscan_closed_form, pin_sscan_reduces_to_ssd, pin_sscan_hand,
            pin_bwd_finite_difference, pin_bwd_transpose, pin_bwd_hand,
            pin_bwd_gated_finite_difference]
