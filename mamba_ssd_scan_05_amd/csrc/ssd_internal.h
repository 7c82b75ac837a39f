// ssd_internal.h -- launch interface between the C ABI (ssd_api.hip) and the
// kernels (ssd_kernels.hip).  Not installed; not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

// Tokens handled per step of a workgroup's walk along a sequence (the
// sub-block on which the quadratic form is evaluated).
constexpr int kSub = 64;

// Parameters of the chunk-walk kernel family.  A workgroup owns one
// (batch, head, segment); the segment covers tokens
// [seg * seg_len, min(L, (seg + 1) * seg_len)).
struct WalkParams {
  const void *x;        // [b, L, H, P]  input dtype
  const float *dt;      // delta_mode 0: raw dt [b, L, H]; 1: Delta [b, H, L]
  const float *dt_bias; // [H] or null (delta_mode 0 only)
  const float *A;       // [H]
  const void *B;        // [b, L, G, N]
  const void *C;        // [b, L, G, N]
  const float *D;       // [H] or null
  const float *init;    // state entering each segment, [(b*H + h)*nseg + seg][P][N]
                        // or null for zero
  void *out;            // [b, L, H, P] or null (state-only walk)
  const void *z;        // [b, L, H, P] gate input (out = y * silu(z)) or null
  float *state_out;     // state leaving each segment, same indexing as init,
                        // or null
  float *final_state;   // [b, H, P, N]: state leaving the last segment, or null
  float *seg_decay;     // [b, H, nseg]: sum of Delta*A*log2(e) over each segment
                        // (state-only walk), or null
  int b, L, H, G, seg_len, nseg;
};

// Walk flavours.
enum WalkMode {
  kWalkFull = 0,      // outputs y; Delta from raw dt (+ bias, softplus)
  kWalkChunkOut = 1,  // outputs y; Delta precomputed [b, H, L]
  kWalkChunkState = 2 // no y; state only; Delta precomputed [b, H, L];
                      // the last segment is skipped (nothing consumes it)
};

hipError_t launch_walk(int dtype, int P, int N, WalkMode mode,
                       const WalkParams &p, hipStream_t stream);

// Whole-sequence quadratic form for L <= kQuadMaxL (ssd_quad.hip): one
// workgroup per (batch, head, 64-token query block); reads x, dt (raw),
// dt_bias, A, B, C, D, init, z and writes out and final_state of p
// (seg_len, nseg, state_out and seg_decay unused).  P in {16, 32, 64} (and
// 128 for bf16), N in {16, 32, 64, 128}.
constexpr int kQuadMaxL = 256;
hipError_t launch_quad(int dtype, int P, int N, const WalkParams &p, hipStream_t stream);

// Parameters of the row-sliced walk (bf16 inputs).  A workgroup of W waves
// owns 16W consecutive state rows -- (head, p) pairs of the heads of one
// group -- of one (batch, group); rows_per_bg = (H/G)*P, wg_per_bg =
// ceil(rows_per_bg / (16W)).
struct RWalkParams {
  const void *x;        // [b, L, H, P] bf16
  const float *dt;      // [b, L, H] raw
  const float *dt_bias; // [H] or null
  const float *A;       // [H]
  const void *B;        // [b, L, G, N] bf16
  const void *C;        // [b, L, G, N] bf16
  const float *D;       // [H] or null
  const void *rec;      // [b, G, ceil(L/64), prep_record_blocks(N), 512] bf16
                        // operand records from launch_prep
  const float *dtT;     // [b, H, 64 ceil(L/64)] step sizes, head-major (launch_prep):
                        // Delta for the plain walk, raw dt for the gated one
  const float *init;    // [b, H, P, N] or null
  void *out;            // [b, L, H, P] bf16
  const void *z;        // [b, L, H, P] bf16 gate input (out = y * silu(z)) or null
  float *final_state;   // [b, H, P, N] or null
  int b, L, H, G, P, rows_per_bg, wg_per_bg;
};

// Operand records of every (batch, group, 64-token sub-block) for the
// row-sliced walk: C, B and causal C_t . B_t' score fragments in matrix-core
// lane order (ssd_prep.hip); prep_record_blocks(N) 1 KiB blocks each.
int prep_record_blocks(int N);
// Also writes the step sizes dt [b, L, H] head-major into dtT [b, H,
// 64 ceil(L/64)]: Delta = softplus(dt + dt_bias [H]) when `softplus` is
// nonzero (dt_bias may be null), the raw dt otherwise.
hipError_t launch_prep(const void *B, const void *C, void *rec, const float *dt, const float *dt_bias, int softplus,
                       float *dtT, int b, int L, int H, int G, int N, hipStream_t stream);

// Row-sliced walk with W waves per workgroup (1..8); N in {32, 64, 128}.
hipError_t launch_rwalk(int N, int W, const RWalkParams &p, hipStream_t stream);

// Step sizes: Delta [b,H,L] = softplus(dt [b,L,H] + dt_bias), head-major.
hipError_t launch_delta(const float *dt, const float *dt_bias, float *delta,
                        int b, int L, int H, hipStream_t stream);

// Inter-chunk state passing over [b,H,nc,P,N] chunk states, in place: slot c
// becomes the state entering chunk c (slot nc-1's own state is not read).
// seg_decay [b,H,nc] holds each chunk's log2 decay.
hipError_t launch_state_pass(float *states, const float *seg_decay,
                             const float *init, int b, int H, int PN, int nc,
                             hipStream_t stream);

// One recurrent step, state in place.
hipError_t launch_step(int dtype, int N, float *state, const void *x,
                       const float *dt, const float *A, const void *B,
                       const void *C, const float *D, void *out, int b, int H,
                       int P, int G, hipStream_t stream);

// Selective scan with a diagonal A per (channel, state index).  A wave owns
// 64 channels of one batch row over one segment of seg_len tokens; channels
// [64k, 64k+64) all read one B/C group (validated on the host).
struct SScanParams {
  const void *x;        // [b, L, Dc]  input dtype
  const float *dt;      // [b, L, Dc]  raw
  const float *dt_bias; // [Dc] or null
  const float *A;       // [Dc, N]
  const void *B;        // [b, L, G, N]
  const void *C;        // [b, L, G, N]
  const float *D;       // [Dc] or null
  const float *init;    // [b, Dc, N] or null
  void *out;            // [b, L, Dc]
  float *final_state;   // [b, Dc, N] or null
  float *hend;          // scratch [b, nseg, Dc, N]: segment end states (nseg > 1)
  float *sdelta;        // scratch [b, nseg, Dc]: sum of Delta per segment
  float *hcopy;         // scratch [b, Dc, N]: staged initial state
  int b, L, Dc, G, seg_len, nseg;
};

// N in {4, 8, 16}; dtype 1 = bf16, 0 = fp32.
hipError_t launch_sscan(int dtype, int N, const SScanParams &p, hipStream_t stream);

// Gradients of the scan (64-token chunks); launch_bwd runs every kernel.
struct BwdParams {
  const void *x;        // [b, L, H, P] input dtype
  const float *dt;      // [b, L, H] raw
  const float *dt_bias; // [H] or null
  const float *A;       // [H]
  const void *B;        // [b, L, G, N]
  const void *C;        // [b, L, G, N]
  const float *D;       // [H] or null
  const void *dy;       // [b, L, H, P] input dtype: gradient at the output
  const float *dfinal;  // [b, H, P, N] or null: gradient at the final state
  const float *states_init; // [b, H, P, N] or null: the initial state
  float *states;        // scratch [b, H, nc, P, N]: state entering each chunk
  float *adj;           // scratch [b, H, nc, P, N]: gradient at each chunk's
                        // last state
  float *part;          // scratch [b, H, nc, 3]: partial dA, dD, d dt_bias
  // the state walks cut into nseg segments of seg_chunks chunks (nseg = 1:
  // one walk over the whole sequence, the arrays below unused)
  float *fpre, *rpre;   // scratch [b, H, nc]: log2 decay from the segment's
                        // start to the chunk (forward) / chunk end to the
                        // segment's end (reverse)
  float *segend_f, *segend_r; // scratch [b, H, nseg, P, N]: segment end states
  float *segdec_f, *segdec_r; // scratch [b, H, nseg]: segment log2 decays
  float *rdec0;         // scratch [b, H]: log2 decay of segment 0
  float *dx;            // [b, L, H, P]
  float *ddt;           // [b, L, H]
  float *dB, *dC;       // [b, L, G, N]
  float *dA;            // [H]
  float *dD, *ddt_bias; // [H] or null
  float *dinit;         // [b, H, P, N] or null
  int b, L, H, G, nc, nseg, seg_chunks;
};
// P in {16, 32, 64}, N in {16, 32, 64, 128}; dtype 1 = bf16, 0 = fp32.
hipError_t launch_bwd(int dtype, int P, int N, const BwdParams &p, hipStream_t stream);
// Gradient through the output gate: dy = dout * silu(z) in the input dtype,
// dz = dout * y * silu'(z) in fp32; n elements, a multiple of 4.
hipError_t launch_gate_bwd(int dtype, const void *y, const void *z, const void *dout, void *dy, float *dz,
                           int64_t n, hipStream_t stream);
} // namespace ssd
