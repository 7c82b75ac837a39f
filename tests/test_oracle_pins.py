"""The fp64 oracle against results fixed independently of it (CPU only)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "ssd_oracle.c")


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_lib, pin):
    pin(oracle_lib)


# Plausible mistakes planted in a copy of the oracle source; every one must be
# caught by at least one pin.  (old text, new text, description)
MUTATIONS = [
    ("double alpha = exp(delta * a_h);", "double alpha = exp(a_h);", "decay without Delta"),
    ("double alpha = exp(delta * a_h);", "double alpha = exp(-delta * a_h);", "decay sign"),
    ("double in = delta * x_t[p];", "double in = x_t[p];", "input gate dropped"),
    ("row[n] = alpha * row[n] + in * B_t[n];\n            acc += row[n] * C_t[n];",
     "row[n] = alpha * row[n] + in * C_t[n];\n            acc += row[n] * B_t[n];",
     "B and C swapped"),
    ("row[n] = alpha * row[n] + in * B_t[n];\n            acc += row[n] * C_t[n];",
     "acc += row[n] * C_t[n];\n            row[n] = alpha * row[n] + in * B_t[n];",
     "readout before update"),
    ("row[n] = alpha * row[n] + in * B_t[n];", "row[n] = alpha * (row[n] + in * B_t[n]);",
     "new input decayed"),
    ("y_t[p] = acc + d_h * x_t[p];", "y_t[p] = acc;", "D term dropped"),
    ("    return m + log1p(exp(-fabs(z)));", "    (void)m;\n    return z;", "no softplus"),
    ("softplus_f64(dt[tok * H + h] + bias);\n            recurrence_token(",
     "softplus_f64(dt[tok * H + h] - bias);\n            recurrence_token(", "bias sign"),
    ("A[h], x + (tok * H + h) * P,", "A[h], x + (tok * H + (H - 1 - h)) * P,", "wrong head of x"),
    ("int64_t g = (h * G) / H;\n        double *S", "int64_t g = h % G;\n        double *S",
     "group map"),
    ("B + (tok * G + g) * N, C + (tok * G + g) * N",
     "B + (tok * G + g) * N, C + ((tok > 0 ? tok - 1 : 0) * G + g) * N", "C one token late"),
    ("recurrence_token(P, N, state + bh * P * N, delta[bh],",
     "recurrence_token(P, N, state + bh * P * N, softplus_f64(delta[bh]),",
     "step applies softplus"),
    ("memcpy(S, init + bh * P * N, (size_t)(P * N) * sizeof(double));",
     "memset(S, 0, (size_t)(P * N) * sizeof(double));", "init ignored"),
    ("out[i] = y[i] * (z[i] / (1.0 + exp(-z[i])));", "out[i] = y[i] * (z[i] / (1.0 + exp(z[i])));",
     "gate logistic sign"),
    ("out[i] = y[i] * (z[i] / (1.0 + exp(-z[i])));", "out[i] = y[i] * (1.0 / (1.0 + exp(-z[i])));",
     "gate sigmoid instead of silu"),
    ("out[i] = y[i] * (z[i] / (1.0 + exp(-z[i])));", "out[i] = (z[i] / (1.0 + exp(-z[i])));",
     "gate drops y"),
    # selective scan (diagonal A per channel and state index)
    ("h[n] = exp(delta * A[d * N + n]) * h[n]", "h[n] = exp(delta * A[n * Dc + d]) * h[n]",
     "selective scan: A transposed"),
    ("h[n] = exp(delta * A[d * N + n]) * h[n]", "h[n] = exp(delta * A[d * N]) * h[n]",
     "selective scan: one A per channel"),
    ("double delta = softplus_f64(dt[tok * Dc + d] + bias);",
     "double delta = softplus_f64(dt[tok * Dc + g] + bias);", "selective scan: Delta of another channel"),
    ("""                h[n] = exp(delta * A[d * N + n]) * h[n] + delta * B_t[n] * xv;
                acc += C_t[n] * h[n];""", """                acc += C_t[n] * h[n];
                h[n] = exp(delta * A[d * N + n]) * h[n] + delta * B_t[n] * xv;""",
     "selective scan: readout before update"),
    ("const double *B_t = B + (tok * G + g) * N, *C_t = C + (tok * G + g) * N;",
     "const double *B_t = C + (tok * G + g) * N, *C_t = B + (tok * G + g) * N;",
     "selective scan: B and C swapped"),
    ("        int64_t g = (d * G) / Dc;\n        double *h", "        int64_t g = d % G;\n        double *h",
     "selective scan: group map"),
    # gradients of the scan
    ("adj[p * N + n] += dyv[p] * Cv[n];", "adj[p * N + n] += dyv[p] * Bv[n] + 0.0 * Cv[n];",
     "backward: adjoint reads B for C"),
    ("dCv[n] += dyv[p] * hv[p * N + n];", "dCv[n] += dyv[p] * hp[p * N + n] + 0.0 * hv[0];",
     "backward: dC from the previous state"),
    ("dx[(tok * H + h) * P + p] = d_h * dyv[p] + delta * gb;",
     "dx[(tok * H + h) * P + p] = 0.0 * d_h + delta * gb;", "backward: dx without the D term"),
    ("d_delta += A[h] * alpha * decay_dot;", "d_delta += alpha * decay_dot;",
     "backward: dDelta decay term without A"),
    ("double ddt_t = d_delta / (1.0 + exp(-z));", "double ddt_t = d_delta + 0.0 * z;",
     "backward: softplus derivative dropped"),
    ("for (int64_t e = 0; e < PN; ++e) adj[e] *= alpha;", "for (int64_t e = 0; e < PN; ++e) adj[e] *= 1.0;",
     "backward: adjoint not decayed"),
    ("dBv[n] += delta * xg;", "dBv[n] += xg;", "backward: dB without Delta"),
    ("part[3 * bh] += delta * alpha * decay_dot;", "part[3 * bh] += alpha * decay_dot;",
     "backward: dA without Delta"),
    ("decay_dot += adj[p * N + n] * hp[p * N + n];", "decay_dot += adj[p * N + n] * hv[p * N + n] + 0.0 * hp[0];",
     "backward: decay term with the current state"),
    ("xg += xv[p] * adj[p * N + n];", "xg += dyv[p] * adj[p * N + n] + 0.0 * xv[0];", "backward: dB from dy"),
    ("dz[i] = dout[i] * y[i] * (sg + z[i] * sg * (1.0 - sg));", "dz[i] = dout[i] * y[i] * sg;",
     "gate backward: silu' taken as the logistic"),
    ("dy[i] = dout[i] * z[i] * sg;", "dy[i] = dout[i] * sg;", "gate backward: dy through the logistic"),
]


@pytest.mark.parametrize("old,new,what", MUTATIONS, ids=[m[2] for m in MUTATIONS])
def test_planted_mistake_is_caught(old, new, what):
    src = open(ORACLE_SRC).read()
    assert src.count(old) == 1, "mutation anchor not found: %s" % what
    tmp = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        path = os.path.join(tmp, "mut.c")
        open(path, "w").write(src.replace(old, new))
        lib = oracle.compile_source(path, os.path.join(tmp, "libmut.so"))
        mutant = oracle.Oracle(lib)
        caught = []
        for pin in pins.ALL_PINS:
            try:
                pin(mutant)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, "planted mistake '%s' passed every pin" % what
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def test_generator_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    from mamba_ssd_scan_05_amd import inputs
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = inputs.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = inputs.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_generator_is_seeded():
    from mamba_ssd_scan_05_amd import inputs
    a = inputs.make_scan(1, 40, 4, 8, 2, 8, seed=7, init_std=0.1)
    b = inputs.make_scan(1, 40, 4, 8, 2, 8, seed=7, init_std=0.1)
    for k in ("x", "dt", "dt_bias", "A", "B", "C", "D", "init"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert np.all(a.A < 0)
