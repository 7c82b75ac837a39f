/*
 * ssd_oracle.c -- fp64 CPU oracle for the Mamba-2 SSD selective scan.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may build, load or call it.  It shares no code, header, table or helper
 * with the HIP library and includes nothing from it.
 *
 * What it computes (written out from the definitions, no chunking, no
 * reordering beyond the plain loops):
 *
 *   Mamba-3 deep dive ch. 2, "SSM foundations" (171host.com), section 2.1.2
 *   (discretization): the discrete recurrence
 *       h_t = exp(Delta_t * A) * h_{t-1} + Delta_t * B_t * x_t
 *   with forget gate alpha_t = exp(Delta_t * A) and input gate gamma_t = Delta_t,
 *   and the readout y_t = C_t^T h_t.  Section 2.1.1 (continuous dynamics) adds
 *   the skip term D * x to the output equation.
 *
 *   Mamba paper-reading notes (sxlin0.github.io), section on the selective
 *   mechanism: Delta = tau_Delta(parameter + s_Delta(x)).  Here the
 *   parameter is dt_bias, s_Delta(x) is the given dt, and tau_Delta is
 *   softplus(z) = log(1 + e^z).
 *
 *   "From Transformer to Mamba" (jsqmd.com), section 2.1: the single-step
 *   shape ssm_step(x_t, h_prev, A, B, C) -> (y_t, h_t).
 *
 *   Gated output (oracle_gate_f64): the Mamba block follows the selective
 *   SSM with a gate before its output projection (Mamba paper-reading
 *   notes, sxlin0.github.io, the section on the simplified block), and the
 *   main branch is a Linear+SiLU ("Transformers are SSMs" summary,
 *   gongshangzheng.github.io, section 2.3, the correspondence table).  Read
 *   as out = y * silu(z), silu(v) = v / (1 + e^{-v}), applied elementwise to
 *   the scan output y (after the D term).
 *
 * Shapes and layouts (all arrays dense, row-major, float64):
 *   x      [b, L, H, P]      dt  [b, L, H]      dt_bias, A, D  [H]
 *   B, C   [b, L, G, N]      heads h use group g = floor(h * G / H)
 *   state  [b, H, P, N]      the per-head state h_t is a P x N matrix whose
 *                            row p is the N-vector state of channel p.
 *
 * Readings where the pages are silent (listed in the design notes as well):
 *   - the initial state enters before the first token's decay, so
 *     h_0 = alpha_0 * init + Delta_0 * B_0 * x_0;
 *   - y_t reads the state after token t has been added (the matrix form's
 *     mask has ones on its diagonal);
 *   - the step call takes Delta itself (already activated), no bias.
 *
 * Parallelism: independent (batch, head) pairs are spread over OpenMP
 * threads; the time loop of each pair is sequential.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(z) = log(1 + exp(z)), evaluated in a form that does not overflow:
 * log(1 + e^z) = max(z, 0) + log1p(exp(-|z|)). */
static double softplus_f64(double z) {
    double m = z > 0.0 ? z : 0.0;
    return m + log1p(exp(-fabs(z)));
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* One token of the recurrence for one (batch, head) pair, in place on S
 * (P x N).  x_t: P values, B_t and C_t: N values.  Writes P outputs. */
static void recurrence_token(int64_t P, int64_t N, double *S, double delta,
                             double a_h, const double *x_t, const double *B_t,
                             const double *C_t, double d_h, double *y_t) {
    double alpha = exp(delta * a_h);           /* forget gate */
    for (int64_t p = 0; p < P; ++p) {
        double *row = S + p * N;
        double in = delta * x_t[p];            /* input gate times input */
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) {
            row[n] = alpha * row[n] + in * B_t[n];
            acc += row[n] * C_t[n];
        }
        y_t[p] = acc + d_h * x_t[p];
    }
}

/* Full-sequence scan.  dt_bias, D and init may be NULL (treated as zero);
 * final_state may be NULL (not written). */
void oracle_scan_f64(int64_t b, int64_t L, int64_t H, int64_t P, int64_t G,
                     int64_t N, const double *x, const double *dt,
                     const double *dt_bias, const double *A, const double *B,
                     const double *C, const double *D, const double *init,
                     double *y, double *final_state) {
    int64_t pairs = b * H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < pairs; ++bh) {
        int64_t ib = bh / H, h = bh % H;
        int64_t g = (h * G) / H;
        double *S = (double *)malloc((size_t)(P * N) * sizeof(double));
        if (init)
            memcpy(S, init + bh * P * N, (size_t)(P * N) * sizeof(double));
        else
            memset(S, 0, (size_t)(P * N) * sizeof(double));
        double bias = dt_bias ? dt_bias[h] : 0.0;
        double d_h = D ? D[h] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            int64_t tok = ib * L + t;
            double delta = softplus_f64(dt[tok * H + h] + bias);
            recurrence_token(P, N, S, delta, A[h], x + (tok * H + h) * P,
                             B + (tok * G + g) * N, C + (tok * G + g) * N, d_h,
                             y + (tok * H + h) * P);
        }
        if (final_state)
            memcpy(final_state + bh * P * N, S, (size_t)(P * N) * sizeof(double));
        free(S);
    }
}

/* One recurrent step for every (batch, head) pair, state updated in place.
 * x [b,H,P], delta [b,H] (already activated), B/C [b,G,N], y [b,H,P]. */
void oracle_step_f64(int64_t b, int64_t H, int64_t P, int64_t G, int64_t N,
                     double *state, const double *x, const double *delta,
                     const double *A, const double *B, const double *C,
                     const double *D, double *y) {
    int64_t pairs = b * H;
#pragma omp parallel for schedule(static)
    for (int64_t bh = 0; bh < pairs; ++bh) {
        int64_t ib = bh / H, h = bh % H;
        int64_t g = (h * G) / H;
        recurrence_token(P, N, state + bh * P * N, delta[bh], A[h], x + bh * P,
                         B + (ib * G + g) * N, C + (ib * G + g) * N,
                         D ? D[h] : 0.0, y + bh * P);
    }
}

/* Gated output: out[i] = y[i] * silu(z[i]), silu(v) = v / (1 + exp(-v)),
 * elementwise over n values. */
void oracle_gate_f64(int64_t n, const double *y, const double *z, double *out) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = y[i] * (z[i] / (1.0 + exp(-z[i])));
}

/* Gradient through the output gate out = y * silu(z) (oracle_gate_f64):
 * dy = dout * silu(z) and dz = dout * y * silu'(z), where
 * silu'(z) = s + z s (1 - s) with s = 1 / (1 + e^{-z}) the logistic. */
void oracle_gate_bwd_f64(int64_t n, const double *y, const double *z, const double *dout,
                         double *dy, double *dz) {
    for (int64_t i = 0; i < n; ++i) {
        double sg = 1.0 / (1.0 + exp(-z[i]));
        dy[i] = dout[i] * z[i] * sg;
        dz[i] = dout[i] * y[i] * (sg + z[i] * sg * (1.0 - sg));
    }
}

/* Selective scan with a per-channel step size and a diagonal A per
 * (channel, state index): the Mamba-1 selective SSM (Mamba paper-reading
 * notes, sxlin0.github.io, the selective-mechanism section: B, C and Delta
 * are functions of the input, Delta = tau_Delta(parameter + s_Delta(x)),
 * applied per channel; the "Transformers are SSMs" summary,
 * gongshangzheng.github.io, section 1.3 table: Mamba-1 keeps a small state,
 * N = 16).  For every batch row and channel d independently:
 *
 *   Delta_t     = softplus(dt[t][d] + dt_bias[d])
 *   h_t[n]      = exp(Delta_t * A[d][n]) * h_{t-1}[n] + Delta_t * B_t[n] * x_t[d]
 *   y_t[d]      = sum_n C_t[n] * h_t[n] + D[d] * x_t[d]
 *
 * Shapes (dense, row-major, float64): x, dt, y [b, L, Dc]; dt_bias, D [Dc];
 * A [Dc, N]; B, C [b, L, G, N] with channel d reading group
 * floor(d * G / Dc); init and final state [b, Dc, N].  dt_bias, D and init
 * may be NULL (zero); final_state may be NULL (not written).  The initial
 * state enters before the first token's decay, as in oracle_scan_f64. */
void oracle_sscan_f64(int64_t b, int64_t L, int64_t Dc, int64_t G, int64_t N,
                      const double *x, const double *dt, const double *dt_bias,
                      const double *A, const double *B, const double *C,
                      const double *D, const double *init, double *y,
                      double *final_state) {
    int64_t pairs = b * Dc;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t bd = 0; bd < pairs; ++bd) {
        int64_t ib = bd / Dc, d = bd % Dc;
        int64_t g = (d * G) / Dc;
        double *h = (double *)malloc((size_t)N * sizeof(double));
        for (int64_t n = 0; n < N; ++n) h[n] = init ? init[bd * N + n] : 0.0;
        double bias = dt_bias ? dt_bias[d] : 0.0;
        double d_d = D ? D[d] : 0.0;
        for (int64_t t = 0; t < L; ++t) {
            int64_t tok = ib * L + t;
            double delta = softplus_f64(dt[tok * Dc + d] + bias);
            double xv = x[tok * Dc + d];
            const double *B_t = B + (tok * G + g) * N, *C_t = C + (tok * G + g) * N;
            double acc = 0.0;
            for (int64_t n = 0; n < N; ++n) {
                h[n] = exp(delta * A[d * N + n]) * h[n] + delta * B_t[n] * xv;
                acc += C_t[n] * h[n];
            }
            y[tok * Dc + d] = acc + d_d * xv;
        }
        if (final_state)
            for (int64_t n = 0; n < N; ++n) final_state[bd * N + n] = h[n];
        free(h);
    }
}

/* Gradients of the full-sequence scan (oracle_scan_f64) by the chain rule,
 * taken through the recurrence one token at a time, latest token first.
 * Training needs them.  The Mamba paper-reading notes (sxlin0.github.io,
 * the section on the hardware-aware selective scan) describe the backward
 * pass as recomputing the states it needs rather than storing them; this
 * checker simply keeps every state of one head in memory.
 *
 * Scalar objective: Lobj = sum_t <dy_t, y_t> + <dfinal, h_{L-1}>, so dy is
 * the gradient arriving at y and dfinal the one arriving at the final state.
 * With z_t = dt_t + dt_bias, Delta_t = softplus(z_t) and
 * alpha_t = exp(Delta_t * A), walking t = L-1 down to 0 with the adjoint
 * g = dLobj/dh_t (P x N, starting from dfinal):
 *
 *   g        += dy_t C_t^T                      (y_t reads h_t)
 *   dC_t     += h_t^T dy_t                      (summed over the group's heads)
 *   dx_t[p]   = D dy_t[p] + Delta_t sum_n g[p][n] B_t[n]
 *   dB_t[n]  += Delta_t sum_p x_t[p] g[p][n]    (summed over the group's heads)
 *   dDelta_t  = sum_{p,n} g[p][n] (A alpha_t h_{t-1}[p][n] + x_t[p] B_t[n])
 *   dA       += Delta_t alpha_t sum_{p,n} g[p][n] h_{t-1}[p][n]
 *   dD       += sum_p dy_t[p] x_t[p]
 *   ddt_t     = dDelta_t * sigmoid(z_t)         (softplus' = sigmoid)
 *   ddt_bias += ddt_t
 *   g         = alpha_t g                       (now dLobj/dh_{t-1})
 *
 * and dinit = g after t = 0.  Shapes as in oracle_scan_f64; dy like y,
 * dfinal like the state (NULL: zero).  Every output is written in full:
 * dx [b,L,H,P], ddt [b,L,H], dA [H], dB and dC [b,L,G,N]; ddt_bias and dD [H]
 * and dinit [b,H,P,N] may be NULL (not written).  Independent (batch, group)
 * pairs run on OpenMP threads; within a pair the group's heads run in order.
 * Per-(batch, head) partial sums of dA, dD and ddt_bias are added over the
 * batch afterwards, in batch order. */
void oracle_scan_bwd_f64(int64_t b, int64_t L, int64_t H, int64_t P, int64_t G,
                         int64_t N, const double *x, const double *dt,
                         const double *dt_bias, const double *A, const double *B,
                         const double *C, const double *D, const double *init,
                         const double *dy, const double *dfinal, double *dx,
                         double *ddt, double *ddt_bias, double *dA, double *dB,
                         double *dC, double *dD, double *dinit) {
    int64_t PN = P * N, hpg = H / G;
    memset(dB, 0, (size_t)(b * L * G * N) * sizeof(double));
    memset(dC, 0, (size_t)(b * L * G * N) * sizeof(double));
    double *part = (double *)calloc((size_t)(3 * b * H), sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < b * G; ++bg) {
        int64_t ib = bg / G, g = bg % G;
        /* hist[t + 1] = hv, hist[0] = the initial state */
        double *hist = (double *)malloc((size_t)((L + 1) * PN) * sizeof(double));
        double *adj = (double *)malloc((size_t)PN * sizeof(double));
        for (int64_t h = g * hpg; h < (g + 1) * hpg; ++h) {
            int64_t bh = ib * H + h;
            double bias = dt_bias ? dt_bias[h] : 0.0;
            double d_h = D ? D[h] : 0.0;
            if (init)
                memcpy(hist, init + bh * PN, (size_t)PN * sizeof(double));
            else
                memset(hist, 0, (size_t)PN * sizeof(double));
            for (int64_t t = 0; t < L; ++t) {       /* forward: every state */
                int64_t tok = ib * L + t;
                double delta = softplus_f64(dt[tok * H + h] + bias);
                double alpha = exp(delta * A[h]);
                const double *xv = x + (tok * H + h) * P, *Bv = B + (tok * G + g) * N;
                const double *prev = hist + t * PN;
                double *cur = hist + (t + 1) * PN;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n)
                        cur[p * N + n] = alpha * prev[p * N + n] + delta * xv[p] * Bv[n];
            }
            if (dfinal)
                memcpy(adj, dfinal + bh * PN, (size_t)PN * sizeof(double));
            else
                memset(adj, 0, (size_t)PN * sizeof(double));
            for (int64_t t = L - 1; t >= 0; --t) {  /* backward */
                int64_t tok = ib * L + t;
                double z = dt[tok * H + h] + bias;
                double delta = softplus_f64(z);
                double alpha = exp(delta * A[h]);
                const double *xv = x + (tok * H + h) * P, *dyv = dy + (tok * H + h) * P;
                const double *Bv = B + (tok * G + g) * N, *Cv = C + (tok * G + g) * N;
                const double *hv = hist + (t + 1) * PN, *hp = hist + t * PN;
                double *dBv = dB + (tok * G + g) * N, *dCv = dC + (tok * G + g) * N;
                for (int64_t p = 0; p < P; ++p)
                    for (int64_t n = 0; n < N; ++n) {
                        adj[p * N + n] += dyv[p] * Cv[n];
                        dCv[n] += dyv[p] * hv[p * N + n];
                    }
                double d_delta = 0.0, decay_dot = 0.0, skip_dot = 0.0;
                for (int64_t p = 0; p < P; ++p) {
                    double gb = 0.0;
                    for (int64_t n = 0; n < N; ++n) {
                        gb += adj[p * N + n] * Bv[n];
                        decay_dot += adj[p * N + n] * hp[p * N + n];
                    }
                    dx[(tok * H + h) * P + p] = d_h * dyv[p] + delta * gb;
                    d_delta += xv[p] * gb;
                    skip_dot += dyv[p] * xv[p];
                }
                for (int64_t n = 0; n < N; ++n) {
                    double xg = 0.0;
                    for (int64_t p = 0; p < P; ++p) xg += xv[p] * adj[p * N + n];
                    dBv[n] += delta * xg;
                }
                d_delta += A[h] * alpha * decay_dot;
                double ddt_t = d_delta / (1.0 + exp(-z));
                ddt[tok * H + h] = ddt_t;
                part[3 * bh] += delta * alpha * decay_dot;
                part[3 * bh + 1] += skip_dot;
                part[3 * bh + 2] += ddt_t;
                for (int64_t e = 0; e < PN; ++e) adj[e] *= alpha;
            }
            if (dinit) memcpy(dinit + bh * PN, adj, (size_t)PN * sizeof(double));
        }
        free(adj);
        free(hist);
    }
    for (int64_t h = 0; h < H; ++h) {
        double sa = 0.0, sd = 0.0, sb = 0.0;
        for (int64_t ib = 0; ib < b; ++ib) {
            sa += part[3 * (ib * H + h)];
            sd += part[3 * (ib * H + h) + 1];
            sb += part[3 * (ib * H + h) + 2];
        }
        dA[h] = sa;
        if (dD) dD[h] = sd;
        if (ddt_bias) ddt_bias[h] = sb;
    }
    free(part);
}
