/*
 * ssd.h -- C ABI of libssd, the Mamba-2 SSD selective scan for AMD MI355X
 * (gfx950).
 *
 * The operation ("Mamba-3 deep dive ch. 2, SSM foundations", 171host.com,
 * section 2.1.2, the discrete recurrence with forget gate alpha and input
 * gate gamma, and section 2.1.1 for the skip term D):
 *
 *     Delta_t = softplus(dt_t + dt_bias_h)
 *     h_t     = exp(Delta_t * A_h) * h_{t-1} + Delta_t * x_t B_t^T   (P x N)
 *     y_t     = h_t C_t + D_h * x_t                                    (P)
 *
 * for every batch row and head h independently; head h reads the B/C group
 * g = floor(h * G / H).  Section 2.2.1 of the same page shows the equal
 * matrix form Y = (L o C B^T) X; the library evaluates it chunk by chunk
 * ("Transformers are SSMs" summary, gongshangzheng.github.io, section 1.2:
 * the quadratic path inside short blocks, the recurrent path across them).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are described by ssd_tensor.  Every tensor must be dense and
 * row-major (strides, in elements, equal to the contiguous strides of its
 * shape) with a 16-byte aligned data pointer.  All data pointers must be
 * memory the current HIP device can address: its own device memory,
 * managed memory, or pinned host memory (read over the bus, slowly).
 * Pageable host memory and another device's memory are refused with
 * SSD_ERR_LAYOUT (checked with hipPointerGetAttributes after every other
 * argument check, before any launch).
 *
 * Ownership: the caller allocates every tensor and keeps it alive until the
 * work queued on `stream` has finished.  The library keeps no pointer to
 * caller memory after a call returns.
 *
 * Scratch: an algorithm that needs scratch space uses a device buffer the
 * library keeps, one per (device, stream) handle, reused by every call on
 * that stream in stream order and grown stream-ordered on `stream` when a
 * call needs more (an event recorded after each call orders the next use if
 * a handle is reused for another stream).  A request above 4 GiB is
 * allocated and freed stream-ordered on `stream` for that call alone.  At
 * most 16 buffers of at most 8 GiB in total are kept: a call that needs a
 * new buffer first frees the least recently used ones (after waiting for
 * their last use) until both limits hold.  Kept buffers live until
 * ssd_release_scratch(), eviction, or the end of the process.  Allocating
 * scratch per call would make the host wait for the stream's earlier work;
 * keeping it lets back-to-back calls queue ahead of the GPU.  Calls that take
 * scratch are serialised on the host while they queue their launches.
 *
 * Errors: every argument is validated on the host before any work is
 * queued; a failed validation returns a nonzero status and queues nothing.  A failed
 * kernel launch or allocation returns SSD_ERR_HIP / SSD_ERR_NOMEM.  Faults
 * inside kernels surface at the caller's next synchronisation.  The text of
 * the most recent error on the calling thread is returned by
 * ssd_last_error().  Calls are asynchronous with respect to the host and
 * ordered on `stream` (a hipStream_t; NULL is the default stream).  No call
 * prints or throws.
 */
#ifndef SSD_H
#define SSD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_VERSION 100 /* 1.0.0 */

/* Element types. */
enum { SSD_F32 = 0, SSD_BF16 = 1 };

/* Status codes. */
enum {
  SSD_OK = 0,
  SSD_ERR_NULL = 1,        /* a required tensor or data pointer is NULL      */
  SSD_ERR_SHAPE = 2,       /* shapes disagree, H % G != 0, b or L is zero    */
  SSD_ERR_DTYPE = 3,       /* unsupported or mismatched element type         */
  SSD_ERR_LAYOUT = 4,      /* not dense row-major, not 16B aligned, or not
                              memory the current device can address        */
  SSD_ERR_UNSUPPORTED = 5, /* P, N, chunk or size outside the supported set  */
  SSD_ERR_ALIAS = 6,       /* an output overlaps an input it may not alias   */
  SSD_ERR_NOMEM = 7,       /* scratch allocation failed                      */
  SSD_ERR_HIP = 8          /* a HIP runtime call or kernel launch failed     */
};

/* Algorithms for ssd_scan_fwd_algo (results agree to rounding). */
enum {
  SSD_ALGO_AUTO = 0,    /* choose by shape                                    */
  SSD_ALGO_FUSED = 1,   /* one kernel; each workgroup walks one (batch, head)
                           sequence in order with the state in registers      */
  SSD_ALGO_CHUNKED = 2, /* chunk-parallel: log-decay cumsum, chunk states,
                           inter-chunk state passing, fused intra+output      */
  SSD_ALGO_ROWS = 3,    /* bf16, N in {32, 64, 128}: C, B and the causal
                           C B^T scores of each (batch, group, 64-token
                           block) laid out once in matrix-core fragment
                           order and shared by the heads of the group; each
                           wave walks 16 state rows of one head            */
  SSD_ALGO_QUAD = 4     /* L <= 256: the whole-sequence quadratic form
                           Y = (L o C B^T) X (+ D x, + the decayed initial
                           state) with no state carried between blocks: one
                           workgroup per (batch, head, 64-token query
                           block), its key blocks spread over its waves;
                           P in {16,32,64} (128 for bf16)                   */
};

/* Dense tensor descriptor.  shape/strides beyond ndim are ignored; strides
 * are in elements. */
typedef struct ssd_tensor {
  void *data;
  int32_t dtype; /* SSD_F32 or SSD_BF16 */
  int32_t ndim;
  int64_t shape[4];
  int64_t strides[4];
} ssd_tensor;

/*
 * ssd_scan_fwd -- forward scan over whole sequences.
 *
 *   x          [b, L, H, P]  f32 or bf16                         required
 *   dt         [b, L, H]     f32, raw (before softplus)           required
 *   dt_bias    [H]           f32, added to dt before softplus     NULL => 0
 *   A          [H]           f32, the decay rate A_h (normally < 0) required
 *   B, C       [b, L, G, N]  dtype of x                           required
 *   D          [H]           f32, skip weight                     NULL => 0
 *   init_state [b, H, P, N]  f32, state before token 0            NULL => 0
 *   out        [b, L, H, P]  dtype of x, written                  required
 *   final_state[b, H, P, N]  f32, state after token L-1           NULL => skip
 *   chunk      a power of two in [64, 65536]: the segment length of the
 *              chunked algorithm, i.e. the granularity at which states are
 *              passed between segments.  A performance knob only: with
 *              SSD_ALGO_AUTO the library chooses the algorithm and segment
 *              length itself (see ssd_scan_plan) and chunk is not used.
 *   stream     hipStream_t
 *
 * The state is stored with N fastest: state[b][h][p][n] is the n-th state
 * entry of channel p (the transpose of the N x P product B x^T).
 * Supported sizes: P in {16, 32, 64, 128} (bf16) or {16, 32, 64} (fp32),
 * N in {16, 32, 64, 128}, H % G == 0, b >= 1, 1 <= L <= 2^24 (any L in
 * that range; the last chunk may be partial), H*P and G*N at most 2^22;
 * larger problems are refused with SSD_ERR_UNSUPPORTED.
 * Arithmetic: products on MFMA in the input dtype with fp32 accumulation,
 * the state and all decay factors in fp32.  final_state may be the same
 * tensor as init_state (updated in place); out may not overlap any input.
 */
int ssd_scan_fwd(const ssd_tensor *x, const ssd_tensor *dt,
                 const ssd_tensor *dt_bias, const ssd_tensor *A,
                 const ssd_tensor *B, const ssd_tensor *C, const ssd_tensor *D,
                 const ssd_tensor *init_state, ssd_tensor *out,
                 ssd_tensor *final_state, int chunk, void *stream);

/* ssd_scan_fwd with an explicit algorithm (SSD_ALGO_*). Same contract;
 * SSD_ALGO_CHUNKED uses `chunk` as its segment length; SSD_ALGO_ROWS
 * returns SSD_ERR_UNSUPPORTED for fp32 inputs or N outside {32, 64, 128}.
 * SSD_ALGO_ROWS and SSD_ALGO_CHUNKED use scratch (see Scratch above; ROWS:
 * b*G*ceil(L/64)*(N/4 + 6) KiB of operand records, 38 KiB per block at
 * N = 128, plus b*H*64*ceil(L/64)*4 bytes for a head-major copy of dt). */
int ssd_scan_fwd_algo(const ssd_tensor *x, const ssd_tensor *dt,
                      const ssd_tensor *dt_bias, const ssd_tensor *A,
                      const ssd_tensor *B, const ssd_tensor *C,
                      const ssd_tensor *D, const ssd_tensor *init_state,
                      ssd_tensor *out, ssd_tensor *final_state, int chunk,
                      int algo, void *stream);

/*
 * ssd_scan_fwd_noalloc -- ssd_scan_fwd for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation.  Same arguments, validation, plan
 * (SSD_ALGO_AUTO) and results as ssd_scan_fwd; the call makes no hipMalloc,
 * hipFree or other allocation.  Its scratch is a fixed array of
 * ssd_fixed_scratch_bytes() bytes (64 MiB) in the library's device memory,
 * one copy per device, held until the process ends; a call whose plan needs
 * more scratch than that returns SSD_ERR_NOMEM before queuing anything
 * (every scratch user writes its scratch before reading it, so nothing
 * needs clearing between calls).  Every ssd_scan_fwd_noalloc call on one
 * device shares that device's array: calls that overlap in time on one
 * device (on different streams, or from several host threads) race on it
 * and must be ordered by the caller.
 */
int ssd_scan_fwd_noalloc(const ssd_tensor *x, const ssd_tensor *dt,
                         const ssd_tensor *dt_bias, const ssd_tensor *A,
                         const ssd_tensor *B, const ssd_tensor *C,
                         const ssd_tensor *D, const ssd_tensor *init_state,
                         ssd_tensor *out, ssd_tensor *final_state, int chunk,
                         void *stream);

/* Size in bytes of the fixed scratch array of ssd_scan_fwd_noalloc. */
int64_t ssd_fixed_scratch_bytes(void);

/*
 * ssd_scan_fwd_gated -- the scan with the block's output gate fused into its
 * output step.  The Mamba block follows the selective SSM with a gate before
 * the output projection (Mamba paper-reading notes, sxlin0.github.io, the
 * section on the simplified block), and its main branch is a Linear+SiLU
 * ("Transformers are SSMs" summary, gongshangzheng.github.io, section 2.3,
 * the correspondence table); read as
 *
 *     out_t = y_t * silu(z_t),   silu(v) = v / (1 + e^{-v})
 *
 * elementwise, with y_t exactly as ssd_scan_fwd computes it (D term
 * included).  final_state is the same as ssd_scan_fwd's.
 *
 *   z   [b, L, H, P]  dtype of x, dense, 16-byte aligned     required
 *
 * Every other argument as ssd_scan_fwd_algo (any algorithm, any supported
 * size).  out and final_state may not overlap z.  Arithmetic: y is formed
 * as in ssd_scan_fwd and the gate in fp32; out is rounded once to the dtype
 * of x, except that SSD_ALGO_ROWS with more than four waves per workgroup
 * rounds y to bf16 before gating (a second rounding of the same size).
 */
int ssd_scan_fwd_gated(const ssd_tensor *x, const ssd_tensor *dt,
                       const ssd_tensor *dt_bias, const ssd_tensor *A,
                       const ssd_tensor *B, const ssd_tensor *C,
                       const ssd_tensor *D, const ssd_tensor *z,
                       const ssd_tensor *init_state, ssd_tensor *out,
                       ssd_tensor *final_state, int chunk, int algo,
                       void *stream);

/*
 * ssd_scan_fwd_rows -- ssd_scan_fwd with SSD_ALGO_ROWS and an explicit
 * workgroup size: `waves` in 1..8 waves per workgroup (16 state rows each),
 * 0 = the size SSD_ALGO_AUTO would take.  For tuning and tests; the result
 * does not depend on `waves` beyond rounding order (it does not at all:
 * every state row is computed by the same instruction sequence).  bf16
 * inputs and N in {32, 64, 128} only (else SSD_ERR_UNSUPPORTED).
 */
int ssd_scan_fwd_rows(const ssd_tensor *x, const ssd_tensor *dt,
                      const ssd_tensor *dt_bias, const ssd_tensor *A,
                      const ssd_tensor *B, const ssd_tensor *C,
                      const ssd_tensor *D, const ssd_tensor *init_state,
                      ssd_tensor *out, ssd_tensor *final_state, int waves,
                      void *stream);

/*
 * ssd_step -- one recurrent step for every (batch, head), state in place
 * ("From Transformer to Mamba", jsqmd.com, section 2.1: the single-step
 * update ssm_step(x_t, h_prev, A, B, C) -> (y_t, h_t); "Mamba-3 deep dive
 * ch. 2", section 2.2.2: recurrent mode with a constant-size cache).
 *
 *   state [b, H, P, N]  f32, read and overwritten with the new state
 *   x     [b, H, P]     f32 or bf16
 *   dt    [b, H]        f32, the step size Delta itself (already activated:
 *                       no bias and no softplus are applied here)
 *   A     [H]           f32                                     required
 *   B, C  [b, G, N]     dtype of x                              required
 *   D     [H]           f32                                     NULL => 0
 *   out   [b, H, P]     dtype of x, written
 *
 * Supported sizes: N in {16, 32, 64, 128, 256}, any P >= 1, H % G == 0.
 * All arithmetic in fp32; out is rounded to its dtype once.  out may not
 * overlap any input or the state.
 */
int ssd_step(ssd_tensor *state, const ssd_tensor *x, const ssd_tensor *dt,
             const ssd_tensor *A, const ssd_tensor *B, const ssd_tensor *C,
             const ssd_tensor *D, ssd_tensor *out, void *stream);

/*
 * ssd_selective_scan_fwd -- the selective scan with a per-channel step size
 * and a diagonal A per (channel, state index), the Mamba-1 selective SSM
 * (Mamba paper-reading notes, sxlin0.github.io, the selective-mechanism
 * section: B, C and Delta depend on the input, Delta per channel; "Transformers
 * are SSMs" summary, gongshangzheng.github.io, section 1.3 table: a small
 * state, N = 16).  For every batch row and channel d:
 *
 *     Delta_t = softplus(dt[t][d] + dt_bias[d])
 *     h_t[n]  = exp(Delta_t * A[d][n]) * h_{t-1}[n] + Delta_t * B_t[n] * x_t[d]
 *     y_t[d]  = sum_n C_t[n] * h_t[n] + D[d] * x_t[d]
 *
 *   x           [b, L, D]     f32 or bf16                        required
 *   dt          [b, L, D]     f32, raw (before bias and softplus) required
 *   dt_bias     [D]           f32                                NULL => 0
 *   A           [D, N]        f32, the values A[d][n]            required
 *   B, C        [b, L, G, N]  dtype of x; channel d reads group
 *                             floor(d * G / D)                   required
 *   D           [D]           f32 (the skip term)                NULL => 0
 *   init_state  [b, D, N]     f32, the state before token 0      NULL => 0
 *   out         [b, L, D]     dtype of x, written
 *   final_state [b, D, N]     f32, written; may be init_state    NULL => skip
 *   segments    the sequence is cut into this many segments walked in
 *               parallel (their entering states folded from a first
 *               state-only pass); 0 chooses from the device size.  Raised
 *               if needed so that one segment's x, dt or out stays under
 *               2 GiB, capped at 1024 and at one segment per 8 tokens.  The
 *               result does not depend on it beyond rounding order.
 *
 * Supported sizes: N in {4, 8, 16}, D/G a multiple of 64 (64 channels of
 * one group per wave), 1 <= L <= 2^24.  The state and all arithmetic in
 * fp32; out is rounded to its dtype once.  Scratch (segment end states,
 * b * segments * D * (N + 1) floats, plus b * D * N staged initial state)
 * is used when segments > 1 (see Scratch above).  out may not overlap any input; final_state may not
 * overlap any input other than (exactly) init_state.
 */
int ssd_selective_scan_fwd(const ssd_tensor *x, const ssd_tensor *dt,
                           const ssd_tensor *dt_bias, const ssd_tensor *A,
                           const ssd_tensor *B, const ssd_tensor *C,
                           const ssd_tensor *D, const ssd_tensor *init_state,
                           ssd_tensor *out, ssd_tensor *final_state,
                           int segments, void *stream);

/*
 * ssd_scan_bwd -- gradients of ssd_scan_fwd with respect to all its inputs.
 *
 * Training needs them.  The Mamba paper-reading notes (sxlin0.github.io, the
 * section on the hardware-aware selective scan) describe the backward pass
 * as recomputing the states it needs instead of storing them.  This call
 * recomputes the states at 64-token chunk boundaries from the inputs and
 * rebuilds everything inside a chunk on chip.  No forward-pass residue is
 * needed.
 *
 * The gradients are those of the scalar sum <dout, y> + <dfinal_state, h_last>,
 * where y and h_last are what ssd_scan_fwd computes from the same inputs.
 * dout is the gradient arriving at the output and dfinal_state the one
 * arriving at the final state.
 *
 * Inputs: x, dt, dt_bias, A, B, C, D and init_state exactly as for
 * ssd_scan_fwd (dt_bias, D, init_state may be NULL: zero).  dout
 * [b,L,H,P] has the dtype of x.  dfinal_state [b,H,P,N] f32 may be NULL
 * (zero).
 *
 * Outputs, all f32, written in full (nothing is accumulated into them):
 *   dx [b,L,H,P]         ddt [b,L,H] (gradient at the raw dt, before
 *                         dt_bias and softplus)
 *   dA [H]               dB, dC [b,L,G,N] (summed over the heads of a group)
 *   ddt_bias [H], dD [H], dinit_state [b,H,P,N]: each may be NULL (not
 *                         computed).
 *
 * Supported: P in {16, 32, 64}, N in {16, 32, 64, 128}, either input dtype,
 * the size limits of ssd_scan_fwd.  No output may overlap an input or another
 * output (SSD_ERR_ALIAS).  Arithmetic: fp32 inputs use fp32 matrix-core
 * products throughout.  bf16 inputs use bf16 matrix-core products with fp32
 * accumulation; where a product pairs a bf16 input with an fp32 quantity
 * (decayed scores, states, adjoints, weighted x or dout), the fp32 operand is
 * carried as a bf16 high part plus a bf16 remainder, so each such product is
 * two bf16 MFMAs with a relative error near 2^-17.  The state walks keep
 * their states in fp32.  Sums over heads, chunks and batch run
 * in a fixed order, so the result does not vary from run to run.  Scratch:
 * b*H*ceil(L/64)*(2*P*N + 3) floats (the states entering each 64-token chunk,
 * the gradients at each chunk's end, per-chunk partial sums; see Scratch
 * above: 1.34 GB at b=4, L=4096, H=80, P=64, N=128, kept between calls
 * like any scratch up to 4 GiB).
 */
int ssd_scan_bwd(const ssd_tensor *x, const ssd_tensor *dt,
                 const ssd_tensor *dt_bias, const ssd_tensor *A,
                 const ssd_tensor *B, const ssd_tensor *C, const ssd_tensor *D,
                 const ssd_tensor *init_state, const ssd_tensor *dout,
                 const ssd_tensor *dfinal_state, ssd_tensor *dx,
                 ssd_tensor *ddt, ssd_tensor *ddt_bias, ssd_tensor *dA,
                 ssd_tensor *dB, ssd_tensor *dC, ssd_tensor *dD,
                 ssd_tensor *dinit_state, void *stream);

/*
 * ssd_scan_bwd_gated -- gradients of ssd_scan_fwd_gated (out = y * silu(z),
 * y the scan output including the D term) for the objective
 * <dout, out> + <dfinal_state, h_last>.
 *
 * The gated output is the Mamba block's gate before its output projection
 * (Mamba paper-reading notes, sxlin0.github.io, the simplified-block section).
 * Arguments are as for ssd_scan_bwd, plus z [b,L,H,P] (dtype of x, an input)
 * and dz [b,L,H,P] f32 (an output, required).  The call recomputes y with the
 * forward scan, forms dy = dout * silu(z) (rounded to x's dtype) and
 * dz = dout * y * silu'(z), then runs ssd_scan_bwd on dy.  Scratch: two
 * tensors the size of x, plus what the forward scan and ssd_scan_bwd use.
 */
int ssd_scan_bwd_gated(const ssd_tensor *x, const ssd_tensor *dt,
                       const ssd_tensor *dt_bias, const ssd_tensor *A,
                       const ssd_tensor *B, const ssd_tensor *C,
                       const ssd_tensor *D, const ssd_tensor *z,
                       const ssd_tensor *init_state, const ssd_tensor *dout,
                       const ssd_tensor *dfinal_state, ssd_tensor *dx,
                       ssd_tensor *ddt, ssd_tensor *ddt_bias, ssd_tensor *dA,
                       ssd_tensor *dB, ssd_tensor *dC, ssd_tensor *dD,
                       ssd_tensor *dz, ssd_tensor *dinit_state, void *stream);

/*
 * ssd_scan_plan -- the plan SSD_ALGO_AUTO uses for a shape on a device with
 * `cus` compute units for inputs of element type `dtype` (SSD_BF16 or
 * SSD_F32), host only, no HIP call: *algo is SSD_ALGO_FUSED,
 * SSD_ALGO_CHUNKED or SSD_ALGO_ROWS and *seg_len the segment length (L for
 * the single-pass walks).
 * The choice trades the spread of (batch, head, segment) walks over the
 * compute units against the extra state-only pass and state traffic of
 * shorter segments.
 */
int ssd_scan_plan(int64_t b, int64_t L, int64_t H, int64_t P, int64_t G,
                  int64_t N, int dtype, int cus, int *algo, int *seg_len);

/* Static text for a status code. */
const char *ssd_status_string(int status);

/* Text of the most recent failure on the calling thread ("" if none). */
const char *ssd_last_error(void);

/* SSD_VERSION of the built library. */
int ssd_version(void);

/* Frees the scratch buffers the library keeps between calls (see Scratch
 * above), after waiting for the queued work that uses them; the next call
 * that needs scratch allocates it again.  Safe to call at any time from any
 * thread (calls that take scratch meanwhile wait for it); returns SSD_OK, or
 * SSD_ERR_HIP if a HIP call failed (the buffers are forgotten either way).
 * Makes no HIP call when no buffer is kept. */
int ssd_release_scratch(void);

/* Number of scratch buffers the library currently keeps and their total
 * bytes (see Scratch above).  Host only; returns SSD_ERR_NULL for a NULL
 * argument. */
int ssd_scratch_stats(int64_t *buffers, int64_t *bytes);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H */
