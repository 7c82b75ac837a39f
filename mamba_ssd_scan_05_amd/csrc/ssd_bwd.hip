// ssd_bwd.hip -- gradients of the SSD scan on MI355X (gfx950).
//
// Training needs the gradients of the scan with respect to all of its
// inputs.  The Mamba paper-reading notes (sxlin0.github.io, the section on
// the hardware-aware selective scan) describe the backward pass as
// recomputing the states it needs instead of keeping them from the forward
// pass; here the states at 64-token chunk boundaries are recomputed by a
// walk over the chunks, and everything inside a chunk is rebuilt on chip.
//
// Notation per (batch, head), chunk of Q = 64 tokens starting at t0, local
// index i: a_i = Delta_i A (log decay), cum_i = a_0 + ... + a_i,
// e_in_i = exp(cum_i), e_out_i = exp(cum_last - cum_i).  H is the state
// entering the chunk, G the gradient arriving at the chunk's last state from
// later tokens and the final state.  Unrolling the recurrence over the chunk
// ("Mamba-3 deep dive ch. 2", section 2.2.1: the mask of the matrix form is
// a product of forget gates) gives, with S = C B^T, E_ij = exp(cum_i - cum_j)
// for i >= j (else 0), M = S o E and DX = dY X^T:
//
//   bracket_t = (M^T dY)_t + e_out_t G B_t            (the adjoint times B_t)
//   dx_t      = D dy_t + Delta_t bracket_t
//   dC_t     += e_in_t H^T dy_t + ((DX o E) diag(Delta) B)_t        (all heads)
//   dB_t     += Delta_t (e_out_t G^T x_t + ((DX o E)^T C)_t)         (all heads)
//   dDelta_t  = x_t . bracket_t + A da_t
//   da_k      = sum_{i >= k > j} W_ij + sum_{i >= k} u_i + sum_{j < k} v_j + w
//
// where W_ij = M_ij DX_ij Delta_j (token j's input reaching output i), u_i =
// e_in_i dy_i . (H C_i) (the entering state reaching output i), v_j =
// e_out_j Delta_j x_j . (G B_j) (input j reaching later tokens) and w =
// exp(cum_last) <G, H>: da_k collects every path whose decay product
// contains a_k.  The first double sum is R_k with R_0 = 0 and
// R_{k+1} = R_k + colsum_k(W) - rowsum_k(W) (W is strictly lower triangular).
//
// The chunk-boundary states H and adjoints G are sequential over chunks:
// H_{c+1} = exp(cum_last^(c)) H_c + sum_j e_out_j Delta_j x_j B_j^T from the
// initial state, and, backwards from the final-state gradient,
// G_{c-1} = exp(cum_last^(c)) G_c + sum_i e_in_i dy_i C_i^T; the gradient of
// the initial state is the last of these, G_{-1}.
//
// Kernels: bwd_state_scan_kernel / _bf16 (both recursions, one workgroup
// per (batch, head) -- or per (batch, head, segment of chunks) when b*H is
// small -- walking the chunks with the state in matrix-core accumulators),
// bwd_fixup_kernel (with segments: adds each segment's carried-in state,
// folded over segments by the state-pass kernel, into its chunks),
// bwd_chunk_kernel / bwd_chunk_bf16_kernel (one workgroup per
// (batch, group, chunk), all heads of the group in turn: dB and dC stay in
// registers across heads, so no atomics and a fixed summation order),
// bwd_param_kernel (sums of the per-(batch, head, chunk) partials of dA, dD
// and d dt_bias), gate_bwd_kernel (the output gate's derivative, for the
// gated call).
//
// Matrix products run on the matrix cores: for fp32 inputs in fp32 (16x16x4
// MFMA) from fp32 LDS tiles; for bf16 inputs in bf16 (16x16x32 MFMA), with
// every fp32 operand carried as a bf16 high part plus a bf16 remainder (the
// _bf16 kernels).
#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kQ = 64;

// Staging of a row of `cols` elements of type T into fp32 LDS, four at a time.
template <typename T>
__device__ __forceinline__ void stage_rows(float *dst, int ld, const T *src, int64_t row_stride, int rows,
                                           int valid_rows, int cols, int tid, int nthreads) {
  const int c4 = cols / 4;
  for (int idx = tid; idx < rows * c4; idx += nthreads) {
    const int r = idx / c4, c = (idx % c4) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < valid_rows) {
      const T *s = src + (int64_t)r * row_stride + c;
      v = make_float4(to_f(s[0]), to_f(s[1]), to_f(s[2]), to_f(s[3]));
    }
    *reinterpret_cast<float4 *>(dst + r * ld + c) = v;
  }
}

// Fragment of a row-major fp32 LDS tile whose K index runs along the row
// (contiguous): row `row`, K-values k0 + {4g .. 4g+3, 16+4g .. 16+4g+3}.
__device__ __forceinline__ FragF32 frag_k_contig(const float *tile, int ld, int row, int k0, int lg) {
  const float *p = tile + row * ld + k0 + 4 * lg;
  return ld4x2(p, p + 16);
}

__device__ __forceinline__ float sum16(float v) { return lane_group_sum<16>(v); } // over a lane group
__device__ __forceinline__ float sum_lg(float v) { // over the 4 lane groups
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}
__device__ __forceinline__ float wave_sum(float v) { return sum_lg(sum16(v)); }
// lane 63's value in every lane (the readlane builtin moves 32-bit integers)
__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Per-chunk decay quantities for one (batch, head), computed by one wave:
// lane k holds token t0 + k.  Returns Delta; writes cum (log2 units), e_in,
// e_out and sigmoid(dt + bias) (the derivative of softplus) for lane k.
struct ChunkDecay {
  float delta, cum2, e_in, e_out, sig, cum2_last;
};
// dt of token t0 + lane of head h (0 past the end of the sequence)
__device__ __forceinline__ float load_dt(const float *dt, int b_, int L, int H, int h, int t0, int lane) {
  const int t = t0 + lane;
  return t < L ? dt[((int64_t)b_ * L + t) * H + h] : 0.f;
}
__device__ __forceinline__ ChunkDecay chunk_decay_v(float dtv, const float *dt_bias, const float *A, int L, int h,
                                                    int t0, int lane) {
  ChunkDecay d;
  const bool valid = t0 + lane < L;
  const float z = valid ? dtv + (dt_bias ? dt_bias[h] : 0.f) : 0.f;
  d.delta = valid ? softplus_f(z) : 0.f;
  d.sig = valid ? __builtin_amdgcn_rcpf(1.f + hw_exp2(-z * kLog2e)) : 0.f;
  d.cum2 = wave_incl_scan(d.delta * A[h] * kLog2e);
  d.cum2_last = lane63(d.cum2);
  d.e_in = hw_exp2(d.cum2);
  d.e_out = hw_exp2(d.cum2_last - d.cum2);
  return d;
}
__device__ __forceinline__ ChunkDecay chunk_decay(const float *dt, const float *dt_bias, const float *A, int b_, int L,
                                                  int H, int h, int t0, int lane) {
  return chunk_decay_v(load_dt(dt, b_, L, H, h, t0, lane), dt_bias, A, L, h, t0, lane);
}

// ---------------------------------------------------------------------------
// Chunk-boundary states of one (batch, head), walking the chunks in order
// with the P x N state held in matrix-core accumulators (4 waves, (P/16) *
// (N/16) 16x16 tiles, wave w owning tiles w, w+4, ...):
//
//   forward (REV = false): S = init; for c = 0 .. nc-1: states[c] = S;
//            S = e_tot_c S + sum_j (e_out_j Delta_j x_j) B_j^T
//   reverse (REV = true):  S = dfinal; for c = nc-1 .. 0: adj[c] = S;
//            S = e_tot_c S + sum_i (e_in_i dy_i) C_i^T;  dinit = S at the end
//
// so states[c] is the state entering chunk c and adj[c] the gradient at
// chunk c's last state (from later tokens and the final state); the final S
// of the reverse walk is the gradient of the initial state.  The next
// chunk's inputs are loaded into registers while the current chunk's
// products run; the per-token weights are applied to the A fragments.

template <typename T, int COLS> struct RowPrefetch {
  // one 64-row tile of COLS elements of T, 16 bytes per load, 256 threads
  static constexpr int kPerRow = COLS * (int)sizeof(T) / 16;
  static constexpr int kLoads = (kQ * kPerRow + 255) / 256;
  uint4 v[kLoads];
  __device__ __forceinline__ void load(const T *src, int64_t row_stride, int valid_rows, int tid) {
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int idx = tid + 256 * k, r = idx / kPerRow, c = idx % kPerRow;
      v[k] = make_uint4(0u, 0u, 0u, 0u);
      if (idx < kQ * kPerRow && r < valid_rows)
        v[k] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(src + (int64_t)r * row_stride) + 16 * c);
    }
  }
  // widen to fp32 rows of `ld` floats
  __device__ __forceinline__ void store(float *dst, int ld, int tid) const {
    constexpr int per16 = 16 / (int)sizeof(T);
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
      const int idx = tid + 256 * k, r = idx / kPerRow, c = idx % kPerRow;
      if (idx >= kQ * kPerRow) continue;
      float *d = dst + r * ld + c * per16;
      if constexpr (sizeof(T) == 2) {
        const __bf16 *e = reinterpret_cast<const __bf16 *>(&v[k]);
#pragma unroll
        for (int q = 0; q < 8; ++q) d[q] = (float)e[q];
      } else {
        *reinterpret_cast<uint4 *>(d) = v[k];
      }
    }
  }
};

template <typename T, int P, int N> struct StateScanLds {
  float sL[kQ * (P + 4)]; // x (forward) or dy (reverse), [token][p]
  float sR[kQ * (N + 4)]; // B (forward) or C (reverse), [token][n]
  float sW[kQ];
  float sTot[1];
};
template <typename T, int P, int N, bool REV>
__device__ __forceinline__ void state_scan_body(const BwdParams &p, int bh, int sg, StateScanLds<T, P, N> &lds) {
  constexpr int LX = P + 4, LB = N + 4, PT = P / 16, NT = N / 16, TILES = (PT * NT + 3) / 4;
  float *sL = lds.sL, *sR = lds.sR, *sW = lds.sW, *sTot = lds.sTot;
  const int nc = p.nc, H = p.H, G = p.G, L = p.L;
  const int b_ = bh / H, h = bh % H, g = (int)(((int64_t)h * G) / H);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int PN = P * N;
  const T *lsrc = reinterpret_cast<const T *>(REV ? p.dy : p.x) + ((int64_t)b_ * L * H + h) * P;
  const T *rsrc = reinterpret_cast<const T *>(REV ? p.C : p.B) + ((int64_t)b_ * L * G + g) * N;
  const float *s0 = REV ? p.dfinal : p.states_init;
  float *out = (REV ? p.adj : p.states) + (int64_t)bh * nc * PN;
  // this workgroup's segment of chunks [c_lo, c_hi).  One segment starts
  // from init (forward) / dfinal (reverse); with several, every segment
  // starts from zero and the fold over segments carries init / dfinal in
  const int nseg = p.nseg, c_lo = sg * p.seg_chunks, c_hi = min(nc, c_lo + p.seg_chunks);
  const int nsteps = c_hi - c_lo;
  const bool from_s0 = nseg == 1;
  float acc_dec = 0.f; // log2 decay walked so far in the segment (wave 0, lane 0)

  f32x4 S[TILES];
#pragma unroll
  for (int k = 0; k < TILES; ++k) {
    const int tile = w + 4 * k, pt = tile % PT, nt = tile / PT;
      if (tile >= PT * NT) break;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[k][r] = (s0 && from_s0) ? s0[(int64_t)bh * PN + (pt * 16 + 4 * lg + r) * N + nt * 16 + li] : 0.f;
  }

  RowPrefetch<T, P> pl;
  RowPrefetch<T, N> pr;
  float dtv = 0.f;
  auto fetch = [&](int c) {
    const int t0 = c * kQ, nv = min(kQ, L - t0);
    pl.load(lsrc + (int64_t)t0 * H * P, (int64_t)H * P, nv, tid);
    pr.load(rsrc + (int64_t)t0 * G * N, (int64_t)G * N, nv, tid);
    if (w == 0) dtv = load_dt(p.dt, b_, L, H, h, t0, lane);
  };
  fetch(REV ? c_hi - 1 : c_lo);
  for (int step = 0; step < nsteps; ++step) {
    const int c = REV ? c_hi - 1 - step : c_lo + step;
    // the state at this chunk boundary
#pragma unroll
    for (int k = 0; k < TILES; ++k) {
      const int tile = w + 4 * k, pt = tile % PT, nt = tile / PT;
      if (tile >= PT * NT) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(int64_t)c * PN + (pt * 16 + 4 * lg + r) * N + nt * 16 + li] = S[k][r];
    }
    pl.store(sL, LX, tid);
    pr.store(sR, LB, tid);
    if (w == 0) {
      const ChunkDecay d = chunk_decay_v(dtv, p.dt_bias, p.A, L, h, c * kQ, lane);
      sW[lane] = REV ? d.e_in : d.e_out * d.delta;
      if (lane == 0) sTot[0] = hw_exp2(d.cum2_last);
      if (lane == 0 && nseg > 1) {
        (REV ? p.rpre : p.fpre)[(int64_t)bh * nc + c] = acc_dec;
        acc_dec += d.cum2_last;
      }
    }
    __syncthreads();
    if (step + 1 < nsteps) fetch(REV ? c - 1 : c + 1);
    const float tot = sTot[0];
    float wk[2][8];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        wk[kk][q] = sW[32 * kk + 4 * lg + q];
        wk[kk][4 + q] = sW[32 * kk + 16 + 4 * lg + q];
      }
#pragma unroll
    for (int k = 0; k < TILES; ++k) {
      const int tile = w + 4 * k, pt = tile % PT, nt = tile / PT;
      if (tile >= PT * NT) break;
      f32x4 acc = S[k] * tot;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        FragF32 a = trfrag(sL, LX, 32 * kk, pt * 16, li, lg);
#pragma unroll
        for (int q = 0; q < 8; ++q) a.v[q] *= wk[kk][q];
        acc = mma(a, trfrag(sR, LB, 32 * kk, nt * 16, li, lg), acc);
      }
      S[k] = acc;
    }
    __syncthreads();
  }
  // the state left at the end of the walk: with one segment, the reverse one
  // is the initial-state gradient; with several, every segment's goes to the
  // fold (reverse segments in reversed order), with the segment's log2 decay,
  // and segment 0's reverse one also to dinit (the fold's carry is added later)
  float *dst0 = nullptr, *dst1 = nullptr;
  if (nseg > 1) {
    const int slot = REV ? nseg - 1 - sg : sg;
    dst0 = (REV ? p.segend_r : p.segend_f) + ((int64_t)bh * nseg + slot) * PN;
    if (w == 0 && lane == 0) {
      (REV ? p.segdec_r : p.segdec_f)[(int64_t)bh * nseg + slot] = acc_dec;
      if (REV && sg == 0) p.rdec0[bh] = acc_dec;
    }
    if (REV && sg == 0 && p.dinit) dst1 = p.dinit + (int64_t)bh * PN;
  } else if (REV && p.dinit) {
    dst0 = p.dinit + (int64_t)bh * PN;
  }
#pragma unroll
  for (int k = 0; k < TILES; ++k) {
    const int tile = w + 4 * k, pt = tile % PT, nt = tile / PT;
    if (tile >= PT * NT) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = (pt * 16 + 4 * lg + r) * N + nt * 16 + li;
      if (dst0) dst0[e] = S[k][r];
      if (dst1) dst1[e] = S[k][r];
    }
  }
}

// Both walks in one launch: blocks [0, b*H*nseg) walk forward, the rest
// backward; block (b*H index) * nseg + segment within each half.
template <typename T, int P, int N>
__global__ void __launch_bounds__(256) bwd_state_scan_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(16))) StateScanLds<T, P, N> lds;
  const int per = p.b * p.H * p.nseg, rem = (int)blockIdx.x % per;
  if ((int)blockIdx.x < per)
    state_scan_body<T, P, N, false>(p, rem / p.nseg, rem % p.nseg, lds);
  else
    state_scan_body<T, P, N, true>(p, rem / p.nseg, rem % p.nseg, lds);
}

// ---------------------------------------------------------------------------
// One workgroup per (batch, group, chunk); 8 waves.  Tile maps (16x16 tiles,
// id -> row tile id % 4, column tile id / 4; wave w takes ids w, w+8, ...):
// every wave owns one row tile (w % 4) of a Q x X product and the column
// tiles w/4, w/4 + 2, ...
template <typename T, int P, int N>
__global__ void __launch_bounds__(512) bwd_chunk_kernel(const BwdParams p) {
  // P or N below 32 run padded to 32 (zero columns/rows in LDS)
  constexpr int PP = P < 32 ? 32 : P, NP = N < 32 ? 32 : N;
  constexpr int LB = NP + 4, LX = PP + 4, LQ = kQ + 4, LS = NP + 4;
  constexpr int PT = PP / 16, NT = NP / 16;
  __shared__ __attribute__((aligned(16))) float sB[kQ * LB];
  __shared__ __attribute__((aligned(16))) float sC[kQ * LB];
  __shared__ __attribute__((aligned(16))) float sX[kQ * LX];
  __shared__ __attribute__((aligned(16))) float sDY[kQ * LX];
  __shared__ __attribute__((aligned(16))) float sM[kQ * LQ];
  __shared__ __attribute__((aligned(16))) float sSt[PP * LS];
  __shared__ float sCum[kQ], sDel[kQ], sEin[kQ], sEout[kQ], sSig[kQ];
  __shared__ float rowW[2][kQ], colW[4][kQ], uP[2][kQ], vP[2][kQ], dinP[2][kQ], sDiag[kQ];
  __shared__ float sRed[9]; // [0]: log2 decay of the chunk; [1 + w]: wave w's share of <G, H>

  const int nc = p.nc, G = p.G, H = p.H, L = p.L;
  const int c = blockIdx.x % nc;
  const int bg = blockIdx.x / nc;
  const int b_ = bg / G, g = bg % G;
  const int hpg = H / G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int rt = w & 3, ct0 = w >> 2;
  const int t0 = c * kQ, nv = min(kQ, L - t0);
  const int PN = P * N;

  if constexpr (PP != P || NP != N) {
    for (int e = tid; e < kQ * LX; e += 512) sX[e] = sDY[e] = 0.f;
    for (int e = tid; e < PP * LS; e += 512) sSt[e] = 0.f;
    for (int e = tid; e < kQ * LB; e += 512) sB[e] = sC[e] = 0.f;
    __syncthreads();
  }

  // B and C of the group's chunk, and S = C B^T (two 16x16 tiles per wave)
  const T *Bg = reinterpret_cast<const T *>(p.B) + (((int64_t)b_ * L + t0) * G + g) * N;
  const T *Cg = reinterpret_cast<const T *>(p.C) + (((int64_t)b_ * L + t0) * G + g) * N;
  stage_rows<T>(sB, LB, Bg, (int64_t)G * N, kQ, nv, N, tid, 512);
  stage_rows<T>(sC, LB, Cg, (int64_t)G * N, kQ, nv, N, tid, 512);
  __syncthreads();
  f32x4 S[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int ct = ct0 + 2 * k;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < NP; k0 += 32)
      acc = mma(frag_k_contig(sC, LB, rt * 16 + li, k0, lg), frag_k_contig(sB, LB, ct * 16 + li, k0, lg), acc);
    S[k] = acc;
  }

  f32x4 dBacc[NT / 2], dCacc[NT / 2];
#pragma unroll
  for (int k = 0; k < NT / 2; ++k) {
    dBacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    dCacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
    const int64_t bh = (int64_t)b_ * H + h;
    const float Ah = p.A[h], Dh = p.D ? p.D[h] : 0.f;
    // --- stage: decays, x, dy, entering state H
    if (w == 0) {
      const ChunkDecay d = chunk_decay(p.dt, p.dt_bias, p.A, b_, L, H, h, t0, lane);
      sCum[lane] = d.cum2;
      sDel[lane] = d.delta;
      sEin[lane] = d.e_in;
      sEout[lane] = d.e_out;
      sSig[lane] = d.sig;
      if (lane == 0) sRed[0] = d.cum2_last;
    }
    const T *xh = reinterpret_cast<const T *>(p.x) + (((int64_t)b_ * L + t0) * H + h) * P;
    const T *dyh = reinterpret_cast<const T *>(p.dy) + (((int64_t)b_ * L + t0) * H + h) * P;
    stage_rows<T>(sX, LX, xh, (int64_t)H * P, kQ, nv, P, tid, 512);
    stage_rows<T>(sDY, LX, dyh, (int64_t)H * P, kQ, nv, P, tid, 512);
    const float *Hs = p.states + (bh * nc + c) * PN;
    for (int idx = tid; idx < PN / 4; idx += 512) {
      const int r = (idx * 4) / N, col = (idx * 4) % N;
      *reinterpret_cast<float4 *>(sSt + r * LS + col) = reinterpret_cast<const float4 *>(Hs)[idx];
    }
    __syncthreads();
    const float cum_last2 = sRed[0];

    // --- DX = dY X^T, M = S o E (to LDS), P2 = DX o E, W sums, diag(DX)
    f32x4 P2[2];
    float rsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ct = ct0 + 2 * k;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < PP; k0 += 32)
        acc = mma(frag_k_contig(sDY, LX, rt * 16 + li, k0, lg), frag_k_contig(sX, LX, ct * 16 + li, k0, lg), acc);
      const int j = ct * 16 + li;
      const float cj = sCum[j], dj = sDel[j];
      float csum = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rt * 16 + 4 * lg + r;
        const float e = (i >= j) ? hw_exp2(sCum[i] - cj) : 0.f;
        const float m = S[k][r] * e;
        sM[i * LQ + j] = m;
        P2[k][r] = acc[r] * e;
        const float wv = (i > j) ? m * acc[r] * dj : 0.f;
        rsum[r] += wv;
        csum += wv;
        if (i == j) sDiag[i] = acc[r];
      }
      csum = sum_lg(csum);
      if (lg == 0) colW[rt][j] = csum;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = sum16(rsum[r]);
      if (li == 0) rowW[ct0][rt * 16 + 4 * lg + r] = v;
    }

    // --- dY H (K = P): dC += e_in o (dY H); u_i = e_in_i sum_n C_in (dY H)_in
    {
      float up[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NT / 2; ++k) {
        const int ct = ct0 + 2 * k;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < PP; k0 += 32)
          acc = mma(frag_k_contig(sDY, LX, rt * 16 + li, k0, lg), trfrag(sSt, LS, k0, ct * 16, li, lg), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = rt * 16 + 4 * lg + r;
          const float v = sEin[i] * acc[r];
          dCacc[k][r] += v;
          up[r] += sC[i * LB + ct * 16 + li] * v;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = sum16(up[r]);
        if (li == 0) uP[ct0][rt * 16 + 4 * lg + r] = v;
      }
    }
    __syncthreads();

    // --- replace H by G (the gradient at the chunk's last state); <G, H>
    {
      const float *Gs = p.adj + (bh * nc + c) * PN;
      float gh = 0.f;
      for (int idx = tid; idx < PN / 4; idx += 512) {
        const int r = (idx * 4) / N, col = (idx * 4) % N;
        float4 *d = reinterpret_cast<float4 *>(sSt + r * LS + col);
        const float4 hv = *d, gv = reinterpret_cast<const float4 *>(Gs)[idx];
        gh += hv.x * gv.x + hv.y * gv.y + hv.z * gv.z + hv.w * gv.w;
        *d = gv;
      }
      gh = wave_sum(gh);
      if (lane == 0) sRed[1 + w] = gh;
    }
    __syncthreads();

    // --- bracket = M^T dY + e_out o (B G^T); dx; x . bracket
    {
      float dp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < PT / 2; ++k) {
        const int ct = ct0 + 2 * k;
        f32x4 a3 = {0.f, 0.f, 0.f, 0.f}, b3 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < kQ; k0 += 32)
          a3 = mma(trfrag(sM, LQ, k0, rt * 16, li, lg), trfrag(sDY, LX, k0, ct * 16, li, lg), a3);
#pragma unroll
        for (int k0 = 0; k0 < NP; k0 += 32)
          b3 = mma(frag_k_contig(sB, LB, rt * 16 + li, k0, lg), frag_k_contig(sSt, LS, ct * 16 + li, k0, lg), b3);
        const int pc = ct * 16 + li;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rt * 16 + 4 * lg + r;
          const float br = a3[r] + sEout[t] * b3[r];
          if (t < nv && pc < P)
            p.dx[(((int64_t)b_ * L + t0 + t) * H + h) * P + pc] = Dh * sDY[t * LX + pc] + sDel[t] * br;
          dp[r] += sX[t * LX + pc] * br;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = sum16(dp[r]);
        if (li == 0) dinP[ct0][rt * 16 + 4 * lg + r] = v;
      }
    }

    // --- X G (K = P): dB part e_out o (X G); v_j = e_out_j Delta_j sum_n B_jn (X G)_jn
    f32x4 acc6[NT / 2];
    {
      float vp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < NT / 2; ++k) {
        const int ct = ct0 + 2 * k;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < PP; k0 += 32)
          acc = mma(frag_k_contig(sX, LX, rt * 16 + li, k0, lg), trfrag(sSt, LS, k0, ct * 16, li, lg), acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = rt * 16 + 4 * lg + r;
          vp[r] += sB[t * LB + ct * 16 + li] * acc[r];
          acc6[k][r] = sEout[t] * acc[r];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = sum16(vp[r]);
        if (li == 0) vP[ct0][rt * 16 + 4 * lg + r] = v;
      }
    }
    __syncthreads();

    // --- P2 = DX o E to LDS; dB += Delta o (e_out o XG + P2^T C)
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) sM[(rt * 16 + 4 * lg + r) * LQ + (ct0 + 2 * k) * 16 + li] = P2[k][r];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NT / 2; ++k) {
      const int ct = ct0 + 2 * k;
      f32x4 acc = acc6[k];
#pragma unroll
      for (int k0 = 0; k0 < kQ; k0 += 32)
        acc = mma(trfrag(sM, LQ, k0, rt * 16, li, lg), trfrag(sC, LB, k0, ct * 16, li, lg), acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) dBacc[k][r] += sDel[rt * 16 + 4 * lg + r] * acc[r];
    }
    __syncthreads();

    // --- P1 = P2 diag(Delta) to LDS; dC += P1 B
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = (ct0 + 2 * k) * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) sM[(rt * 16 + 4 * lg + r) * LQ + j] = P2[k][r] * sDel[j];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NT / 2; ++k) {
      const int ct = ct0 + 2 * k;
      f32x4 acc = dCacc[k];
#pragma unroll
      for (int k0 = 0; k0 < kQ; k0 += 32)
        acc = mma(frag_k_contig(sM, LQ, rt * 16 + li, k0, lg), trfrag(sB, LB, k0, ct * 16, li, lg), acc);
      dCacc[k] = acc;
    }

    // --- da, ddt and the head's partial sums (wave 0, lane k = token)
    if (w == 0) {
      const int k = lane;
      const float colsum = colW[0][k] + colW[1][k] + colW[2][k] + colW[3][k];
      const float rowsum = rowW[0][k] + rowW[1][k];
      const float dlt = colsum - rowsum;
      const float R = wave_incl_scan(dlt) - dlt;           // sum over m < k
      const float u = uP[0][k] + uP[1][k];
      const float u_incl = wave_incl_scan(u);
      const float U = lane63(u_incl) - u_incl + u;  // sum over i >= k
      const float v = sEout[k] * sDel[k] * (vP[0][k] + vP[1][k]);
      const float V = wave_incl_scan(v) - v;               // sum over j < k
      float gh = 0.f;
#pragma unroll
      for (int q = 1; q <= 8; ++q) gh += sRed[q];
      const float da = R + U + V + hw_exp2(cum_last2) * gh;
      const float din = dinP[0][k] + dinP[1][k];
      const float ddt = (din + Ah * da) * sSig[k];
      const bool valid = k < nv;
      if (valid) p.ddt[((int64_t)b_ * L + t0 + k) * H + h] = ddt;
      const float pa = wave_sum(valid ? sDel[k] * da : 0.f);
      const float pd = wave_sum(valid ? sDiag[k] : 0.f);
      const float pb = wave_sum(valid ? ddt : 0.f);
      if (lane == 0) {
        float *q = p.part + (bh * nc + c) * 3;
        q[0] = pa;
        q[1] = pd;
        q[2] = pb;
      }
    }
    __syncthreads();
  }

  // dB, dC of the group's chunk (fp32)
#pragma unroll
  for (int k = 0; k < NT / 2; ++k) {
    const int n = (ct0 + 2 * k) * 16 + li;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = rt * 16 + 4 * lg + r;
      if (t < nv && n < N) {
        const int64_t o = (((int64_t)b_ * L + t0 + t) * G + g) * N + n;
        p.dB[o] = dBacc[k][r];
        p.dC[o] = dCacc[k][r];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The same chunk step for bf16 inputs on the bf16 matrix cores.  Every
// product pairs an input operand (x, dy, B or C: exact in bf16) with either
// another input or an fp32 quantity (M, DX o E, the states H and G).  An
// fp32 operand v is kept in LDS as two bf16 planes, hi = bf16(v) and
// lo = bf16(v - hi), and each product is two bf16 MFMAs, input * hi +
// input * lo, accumulated in fp32: relative error at most about 2^-18 per
// product (lo carries the next 8 bits of v), against 2^-24 for fp32 MFMA,
// at a quarter of the matrix-core time.  Tile maps as in bwd_chunk_kernel.
__device__ __forceinline__ void put_split(__bf16 *hi, __bf16 *lo, int off, float v) {
  const __bf16 h = (__bf16)v;
  hi[off] = h;
  lo[off] = (__bf16)(v - (float)h);
}
__device__ __forceinline__ FragBF kc16(const __bf16 *tile, int ld, int row, int k0, int lg) {
  const __bf16 *p = tile + row * ld + k0 + 4 * lg;
  return ld4x2(p, p + 16);
}
// copy `rows` rows of `cols` bf16 (16 B at a time), zero rows >= valid_rows
__device__ __forceinline__ void stage_bf16(__bf16 *dst, int ld, const __bf16 *src, int64_t row_stride, int rows,
                                           int valid_rows, int cols, int tid, int nthreads) {
  const int c8 = cols / 8;
  for (int idx = tid; idx < rows * c8; idx += nthreads) {
    const int r = idx / c8, c = (idx % c8) * 8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < valid_rows) v = *reinterpret_cast<const uint4 *>(src + (int64_t)r * row_stride + c);
    *reinterpret_cast<uint4 *>(dst + r * ld + c) = v;
  }
}
// fp32 P x N state from global into hi/lo planes; returns this thread's share
// of <state, other> when `other` is given (exact fp32 values from global)
template <int N>
__device__ __forceinline__ float stage_state_split(__bf16 *hi, __bf16 *lo, int ld, const float *src,
                                                   const float *other, int PN, int tid, int nthreads) {
  float dot = 0.f;
  for (int idx = tid; idx < PN / 4; idx += nthreads) {
    const int r = (idx * 4) / N, col = (idx * 4) % N;
    const float4 v = reinterpret_cast<const float4 *>(src)[idx];
    if (other) {
      const float4 o = reinterpret_cast<const float4 *>(other)[idx];
      dot += v.x * o.x + v.y * o.y + v.z * o.z + v.w * o.w;
    }
    const int off = r * ld + col;
    put_split(hi, lo, off, v.x);
    put_split(hi, lo, off + 1, v.y);
    put_split(hi, lo, off + 2, v.z);
    put_split(hi, lo, off + 3, v.w);
  }
  return dot;
}

// The same walk for bf16 inputs on the bf16 matrix cores: the weighted
// input w_j x_j (fp32) is kept as a bf16 high part plus a bf16 remainder,
// B or C are exact in bf16, and each product is two 16x16x32 MFMAs.
template <int P, int N> struct StateScanBf16Lds {
  __bf16 sLh[kQ * tr_ld(P, 2)];
  __bf16 sLl[kQ * tr_ld(P, 2)];
  __bf16 sR[kQ * tr_ld(N, 2)];
  float sW[kQ];
  float sTot[1];
};
template <int P, int N, bool REV>
__device__ __forceinline__ void state_scan_bf16_body(const BwdParams &p, int bh, int sg, StateScanBf16Lds<P, N> &lds) {
  constexpr int LX = tr_ld(P, 2), LB = tr_ld(N, 2), PT = P / 16, NT = N / 16, TILES = (PT * NT + 3) / 4;
  __bf16 *sLh = lds.sLh, *sLl = lds.sLl, *sR = lds.sR;
  float *sW = lds.sW, *sTot = lds.sTot;
  const int nc = p.nc, H = p.H, G = p.G, L = p.L;
  const int b_ = bh / H, h = bh % H, g = (int)(((int64_t)h * G) / H);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int PN = P * N;
  const __bf16 *lsrc = reinterpret_cast<const __bf16 *>(REV ? p.dy : p.x) + ((int64_t)b_ * L * H + h) * P;
  const __bf16 *rsrc = reinterpret_cast<const __bf16 *>(REV ? p.C : p.B) + ((int64_t)b_ * L * G + g) * N;
  const float *s0 = REV ? p.dfinal : p.states_init;
  float *out = (REV ? p.adj : p.states) + (int64_t)bh * nc * PN;
  // this workgroup's segment of chunks [c_lo, c_hi).  One segment starts
  // from init (forward) / dfinal (reverse); with several, every segment
  // starts from zero and the fold over segments carries init / dfinal in
  const int nseg = p.nseg, c_lo = sg * p.seg_chunks, c_hi = min(nc, c_lo + p.seg_chunks);
  const int nsteps = c_hi - c_lo;
  const bool from_s0 = nseg == 1;
  float acc_dec = 0.f; // log2 decay walked so far in the segment (wave 0, lane 0)

  f32x4 S[TILES];
#pragma unroll
  for (int k = 0; k < TILES; ++k) {
    const int tile = w + 4 * k, pt = tile % PT, nt = tile / PT;
      if (tile >= PT * NT) break;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      S[k][r] = (s0 && from_s0) ? s0[(int64_t)bh * PN + (pt * 16 + 4 * lg + r) * N + nt * 16 + li] : 0.f;
  }

  RowPrefetch<__bf16, P> pl;
  RowPrefetch<__bf16, N> pr;
  float dtv = 0.f;
  auto fetch = [&](int c) {
    const int t0 = c * kQ, nv = min(kQ, L - t0);
    pl.load(lsrc + (int64_t)t0 * H * P, (int64_t)H * P, nv, tid);
    pr.load(rsrc + (int64_t)t0 * G * N, (int64_t)G * N, nv, tid);
    if (w == 0) dtv = load_dt(p.dt, b_, L, H, h, t0, lane);
  };
  fetch(REV ? c_hi - 1 : c_lo);
  for (int step = 0; step < nsteps; ++step) {
    const int c = REV ? c_hi - 1 - step : c_lo + step;
#pragma unroll
    for (int k = 0; k < TILES; ++k) {
      const int tile = w + 4 * k, pt = tile % PT, nt = tile / PT;
      if (tile >= PT * NT) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(int64_t)c * PN + (pt * 16 + 4 * lg + r) * N + nt * 16 + li] = S[k][r];
    }
    if (w == 0) {
      const ChunkDecay d = chunk_decay_v(dtv, p.dt_bias, p.A, L, h, c * kQ, lane);
      sW[lane] = REV ? d.e_in : d.e_out * d.delta;
      if (lane == 0) sTot[0] = hw_exp2(d.cum2_last);
      if (lane == 0 && nseg > 1) {
        (REV ? p.rpre : p.fpre)[(int64_t)bh * nc + c] = acc_dec;
        acc_dec += d.cum2_last;
      }
    }
    __syncthreads();
    // stage: weighted input split into hi/lo planes, B or C copied
    {
      constexpr int KP = RowPrefetch<__bf16, P>::kPerRow;
#pragma unroll
      for (int k = 0; k < RowPrefetch<__bf16, P>::kLoads; ++k) {
        const int idx = tid + 256 * k, r = idx / KP, cc = idx % KP;
        if (idx >= kQ * KP) continue;
        const __bf16 *e = reinterpret_cast<const __bf16 *>(&pl.v[k]);
        const float wr = sW[r];
        bf16x8 hv, lv;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float v = wr * (float)e[q];
          hv[q] = (__bf16)v;
          lv[q] = (__bf16)(v - (float)hv[q]);
        }
        // eight consecutive values of a row: one 16-byte write per plane
        *reinterpret_cast<bf16x8 *>(sLh + r * LX + cc * 8) = hv;
        *reinterpret_cast<bf16x8 *>(sLl + r * LX + cc * 8) = lv;
      }
      constexpr int KN = RowPrefetch<__bf16, N>::kPerRow;
#pragma unroll
      for (int k = 0; k < RowPrefetch<__bf16, N>::kLoads; ++k) {
        const int idx = tid + 256 * k, r = idx / KN, cc = idx % KN;
        if (idx >= kQ * KN) continue;
        *reinterpret_cast<uint4 *>(sR + r * LB + cc * 8) = pr.v[k];
      }
    }
    const float tot = sTot[0];
    __syncthreads();
    if (step + 1 < nsteps) fetch(REV ? c - 1 : c + 1);
#pragma unroll
    for (int k = 0; k < TILES; ++k) {
      const int tile = w + 4 * k, pt = tile % PT, nt = tile / PT;
      if (tile >= PT * NT) break;
      f32x4 acc = S[k] * tot;
#pragma unroll
      for (int k0 = 0; k0 < kQ; k0 += 32) {
        const FragBF bb = trfrag(sR, LB, k0, nt * 16, li, lg);
        acc = mma(trfrag(sLh, LX, k0, pt * 16, li, lg), bb, acc);
        acc = mma(trfrag(sLl, LX, k0, pt * 16, li, lg), bb, acc);
      }
      S[k] = acc;
    }
    __syncthreads();
  }
  // the state left at the end of the walk: with one segment, the reverse one
  // is the initial-state gradient; with several, every segment's goes to the
  // fold (reverse segments in reversed order), with the segment's log2 decay,
  // and segment 0's reverse one also to dinit (the fold's carry is added later)
  float *dst0 = nullptr, *dst1 = nullptr;
  if (nseg > 1) {
    const int slot = REV ? nseg - 1 - sg : sg;
    dst0 = (REV ? p.segend_r : p.segend_f) + ((int64_t)bh * nseg + slot) * PN;
    if (w == 0 && lane == 0) {
      (REV ? p.segdec_r : p.segdec_f)[(int64_t)bh * nseg + slot] = acc_dec;
      if (REV && sg == 0) p.rdec0[bh] = acc_dec;
    }
    if (REV && sg == 0 && p.dinit) dst1 = p.dinit + (int64_t)bh * PN;
  } else if (REV && p.dinit) {
    dst0 = p.dinit + (int64_t)bh * PN;
  }
#pragma unroll
  for (int k = 0; k < TILES; ++k) {
    const int tile = w + 4 * k, pt = tile % PT, nt = tile / PT;
    if (tile >= PT * NT) break;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int e = (pt * 16 + 4 * lg + r) * N + nt * 16 + li;
      if (dst0) dst0[e] = S[k][r];
      if (dst1) dst1[e] = S[k][r];
    }
  }
}

template <int P, int N>
__global__ void __launch_bounds__(256) bwd_state_scan_bf16_kernel(const BwdParams p) {
  __shared__ __attribute__((aligned(16))) StateScanBf16Lds<P, N> lds;
  const int per = p.b * p.H * p.nseg, rem = (int)blockIdx.x % per;
  if ((int)blockIdx.x < per)
    state_scan_bf16_body<P, N, false>(p, rem / p.nseg, rem % p.nseg, lds);
  else
    state_scan_bf16_body<P, N, true>(p, rem / p.nseg, rem % p.nseg, lds);
}

// Chunk step body for NW waves.  A wave owns U = 8 / NW of the four 16-token
// row tiles (rt0 .. rt0 + U - 1) and the column tiles ct0, ct0 + 2, ...;
// inside each product the loop over its row tiles is innermost, so a
// fragment along the other operand is read once for all of them.  The
// kernel runs NW = 8 (two waves per SIMD, 256 VGPRs each); NW = 4 (one wave
// per SIMD, up to 512 registers with the accumulators in AGPRs, two row
// tiles per wave) gives the same results and measured 1.73 ms against
// 1.36 ms for the whole backward at the 2.7B layer shape: one wave per
// SIMD leaves the LDS and memory latency exposed.
template <int P, int N, int NW>
__device__ __forceinline__ void chunk_bf16_body(const BwdParams &p) {
  // P or N below 32 run padded to 32 (zero columns/rows in LDS)
  constexpr int PP = P < 32 ? 32 : P, NP = N < 32 ? 32 : N;
  constexpr int LB = tr_ld(NP, 2), LX = tr_ld(PP, 2), LQ = tr_ld(kQ, 2), LS = tr_ld(NP, 2);
  constexpr int PT = PP / 16, NT = NP / 16;
  constexpr int NTH = NW * 64, U = 8 / NW, RG = 4 / U;
  static_assert(NW == 8 || NW == 4, "8 or 4 waves");
  __shared__ __attribute__((aligned(16))) __bf16 sB[kQ * LB];
  __shared__ __attribute__((aligned(16))) __bf16 sC[kQ * LB];
  __shared__ __attribute__((aligned(16))) __bf16 sX[kQ * LX];
  __shared__ __attribute__((aligned(16))) __bf16 sDY[kQ * LX];
  __shared__ __attribute__((aligned(16))) __bf16 sMh[kQ * LQ];
  __shared__ __attribute__((aligned(16))) __bf16 sMl[kQ * LQ];
  __shared__ __attribute__((aligned(16))) __bf16 sSh[PP * LS];
  __shared__ __attribute__((aligned(16))) __bf16 sSl[PP * LS];
  // G of the coming head, fp32 [P][N], copied straight from global memory to
  // LDS (buffer loads to LDS, 1 KiB per wave instruction) ahead of its use
  __shared__ __attribute__((aligned(16))) float sGst[P * N];
  // per-token decay quantities, double-buffered: the next head's are formed
  // while the current head finishes
  __shared__ float sCumB[2][kQ], sDelB[2][kQ], sEinB[2][kQ], sEoutB[2][kQ], sSigB[2][kQ];
  __shared__ float rowW[2][kQ], colW[4][kQ], uP[2][kQ], vP[2][kQ], dinP[2][kQ], sDiag[kQ];
  __shared__ float sRed[1 + NW]; // [1 + w]: wave w's share of <G, H>
  __shared__ float sLast[2];     // log2 decay of the chunk, per decay buffer

  const int nc = p.nc, G = p.G, H = p.H, L = p.L;
  const int c = blockIdx.x % nc;
  const int bg = blockIdx.x / nc;
  const int b_ = bg / G, g = bg % G;
  const int hpg = H / G;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, li = lane & 15, lg = lane >> 4;
  const int rt0 = (w % RG) * U, ct0 = w / RG;
  const int t0 = c * kQ, nv = min(kQ, L - t0);
  const int PN = P * N;

  if constexpr (PP != P || NP != N) {
    for (int e = tid; e < kQ * LX; e += NTH) sX[e] = sDY[e] = (__bf16)0.f;
    for (int e = tid; e < PP * LS; e += NTH) sSh[e] = sSl[e] = (__bf16)0.f;
    for (int e = tid; e < kQ * LB; e += NTH) sB[e] = sC[e] = (__bf16)0.f;
    lds_barrier();
  }

  const __bf16 *Bg = reinterpret_cast<const __bf16 *>(p.B) + (((int64_t)b_ * L + t0) * G + g) * N;
  const __bf16 *Cg = reinterpret_cast<const __bf16 *>(p.C) + (((int64_t)b_ * L + t0) * G + g) * N;
  stage_bf16(sB, LB, Bg, (int64_t)G * N, kQ, nv, N, tid, NTH);
  stage_bf16(sC, LB, Cg, (int64_t)G * N, kQ, nv, N, tid, NTH);
  lds_barrier();
  f32x4 S[U][2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int ct = ct0 + 2 * k;
#pragma unroll
    for (int u = 0; u < U; ++u) S[u][k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k0 = 0; k0 < NP; k0 += 32) {
      const FragBF bb = kc16(sB, LB, ct * 16 + li, k0, lg);
#pragma unroll
      for (int u = 0; u < U; ++u) S[u][k] = mma(kc16(sC, LB, (rt0 + u) * 16 + li, k0, lg), bb, S[u][k]);
    }
  }

  f32x4 dBacc[U][NT / 2], dCacc[U][NT / 2];
#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int k = 0; k < NT / 2; ++k) {
      dBacc[u][k] = f32x4{0.f, 0.f, 0.f, 0.f};
      dCacc[u][k] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  // decays of head hh into buffer q (one wave), and x, dy, the entering state
  // of head hh into LDS (threads [t_lo, t_lo + nt))
  auto decay_of = [&](int hh, int q) {
    const ChunkDecay d = chunk_decay(p.dt, p.dt_bias, p.A, b_, L, H, hh, t0, lane);
    sCumB[q][lane] = d.cum2;
    sDelB[q][lane] = d.delta;
    sEinB[q][lane] = d.e_in;
    sEoutB[q][lane] = d.e_out;
    sSigB[q][lane] = d.sig;
    if (lane == 0) sLast[q] = d.cum2_last;
  };
  auto stage_head = [&](int hh, int t_lo, int nt) {
    const __bf16 *xh = reinterpret_cast<const __bf16 *>(p.x) + (((int64_t)b_ * L + t0) * H + hh) * P;
    const __bf16 *dyh = reinterpret_cast<const __bf16 *>(p.dy) + (((int64_t)b_ * L + t0) * H + hh) * P;
    stage_bf16(sX, LX, xh, (int64_t)H * P, kQ, nv, P, tid - t_lo, nt);
    stage_bf16(sDY, LX, dyh, (int64_t)H * P, kQ, nv, P, tid - t_lo, nt);
    stage_state_split<N>(sSh, sSl, LS, p.states + (((int64_t)b_ * H + hh) * nc + c) * PN, nullptr, PN,
                         tid - t_lo, nt);
  };
  // G of head hh into sGst: 1 KiB pieces q = w - w_lo, w - w_lo + nw, ...
  auto fetch_g = [&](int hh, int w_lo, int nw) {
    const float *Gn = p.adj + (((int64_t)b_ * H + hh) * nc + c) * PN;
    const auto rs = make_rsrc(Gn, (uint32_t)PN * 4u);
    for (int q = w - w_lo; q < PN / 256; q += nw)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(sGst + q * 256), 16,
                                               q * 1024 + lane * 16, 0, 0, 0);
  };
  // the entering state of head hh into sGst (fp32, 1 KiB pieces as fetch_g)
  auto fetch_h = [&](int hh, int w_lo, int nw) {
    const float *Hn = p.states + (((int64_t)b_ * H + hh) * nc + c) * PN;
    const auto rs = make_rsrc(Hn, (uint32_t)PN * 4u);
    for (int q = w - w_lo; q < PN / 256; q += nw)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void *)(sGst + q * 256), 16,
                                               q * 1024 + lane * 16, 0, 0, 0);
  };
  // this thread's 16-byte pieces (tid, tid + NTH, ...) of the next head's x
  // and dy (tokens past the end read zero): loaded into registers during the
  // dB / dC products, written to LDS in the tail
  constexpr int XPC = P / 8, NXP = kQ * XPC, NPC = (NXP + NTH - 1) / NTH;
  if (w == 0) decay_of(g * hpg, 0);
  stage_head(g * hpg, 0, NTH);
  fetch_g(g * hpg, 0, NW);
  lds_barrier();

  for (int h = g * hpg; h < (g + 1) * hpg; ++h) {
    const int64_t bh = (int64_t)b_ * H + h;
    const float Ah = p.A[h], Dh = p.D ? p.D[h] : 0.f;
    const int cur = (h - g * hpg) & 1;
    float *sCum = sCumB[cur], *sDel = sDelB[cur], *sEin = sEinB[cur], *sEout = sEoutB[cur], *sSig = sSigB[cur];
    const float cum_last2 = sLast[cur];

    // --- DX = dY X^T, M = S o E (split to LDS), P2 = DX o E, W sums, diag(DX)
    f32x4 P2[U][2];
    float rsum[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) rsum[u][r] = 0.f;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int ct = ct0 + 2 * k;
      f32x4 acc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < PP; k0 += 32) {
        const FragBF bx = kc16(sX, LX, ct * 16 + li, k0, lg);
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = mma(kc16(sDY, LX, (rt0 + u) * 16 + li, k0, lg), bx, acc[u]);
      }
      const int j = ct * 16 + li;
      const float cj = sCum[j], dj = sDel[j];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int rt = rt0 + u;
        float csum = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = rt * 16 + 4 * lg + r;
          const float e = (i >= j) ? hw_exp2(sCum[i] - cj) : 0.f;
          const float m = S[u][k][r] * e;
          put_split(sMh, sMl, i * LQ + j, m);
          P2[u][k][r] = acc[u][r] * e;
          const float wv = (i > j) ? m * acc[u][r] * dj : 0.f;
          rsum[u][r] += wv;
          csum += wv;
          if (i == j) sDiag[i] = acc[u][r];
        }
        csum = sum_lg(csum);
        if (lg == 0) colW[rt][j] = csum;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = sum16(rsum[u][r]);
        if (li == 0) rowW[ct0][(rt0 + u) * 16 + 4 * lg + r] = v;
      }

    // --- dY H: dC += e_in o (dY H); u_i = e_in_i sum_n C_in (dY H)_in
    {
      float up[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) up[u][r] = 0.f;
#pragma unroll
      for (int k = 0; k < NT / 2; ++k) {
        const int ct = ct0 + 2 * k;
        f32x4 acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < PP; k0 += 32) {
          const FragBF bh = trfrag(sSh, LS, k0, ct * 16, li, lg), bl = trfrag(sSl, LS, k0, ct * 16, li, lg);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const FragBF a = kc16(sDY, LX, (rt0 + u) * 16 + li, k0, lg);
            acc[u] = mma(a, bh, acc[u]);
            acc[u] = mma(a, bl, acc[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = (rt0 + u) * 16 + 4 * lg + r;
            const float v = sEin[i] * acc[u][r];
            dCacc[u][k][r] += v;
            up[u][r] += (float)sC[i * LB + ct * 16 + li] * v;
          }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = sum16(up[u][r]);
          if (li == 0) uP[ct0][(rt0 + u) * 16 + 4 * lg + r] = v;
        }
    }
    // every wave is done with H's planes, and its copy of G into sGst has
    // landed (each wave waits for its own copies before the barrier)
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();

    // --- replace H by G (already in LDS); <G, H> with H from its two planes
    {
      float gh = 0.f;
      for (int idx = tid; idx < PN / 4; idx += NTH) {
        const int r = (idx * 4) / N, col = (idx * 4) % N, off = r * LS + col;
        const float4 gv = *reinterpret_cast<const float4 *>(sGst + 4 * idx);
        const float gq[4] = {gv.x, gv.y, gv.z, gv.w};
        // four consecutive columns: 8-byte reads and writes per plane
        const bf16x4 oh = *reinterpret_cast<const bf16x4 *>(sSh + off), ol = *reinterpret_cast<const bf16x4 *>(sSl + off);
        bf16x4 nh, nl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          gh += gq[q] * ((float)oh[q] + (float)ol[q]);
          nh[q] = (__bf16)gq[q];
          nl[q] = (__bf16)(gq[q] - (float)nh[q]);
        }
        *reinterpret_cast<bf16x4 *>(sSh + off) = nh;
        *reinterpret_cast<bf16x4 *>(sSl + off) = nl;
      }
      gh = wave_sum(gh);
      if (lane == 0) sRed[1 + w] = gh;
    }
    lds_barrier();
    // sGst is free until the tail: copy the next head's entering state into it
    const bool has_next = h + 1 < (g + 1) * hpg;
    if (has_next && w >= 2) fetch_h(h + 1, 2, NW - 2);

    // --- bracket = M^T dY + e_out o (B G^T); dx; x . bracket
    {
      float dp[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) dp[u][r] = 0.f;
#pragma unroll
      for (int k = 0; k < PT / 2; ++k) {
        const int ct = ct0 + 2 * k;
        f32x4 a3[U], b3[U];
#pragma unroll
        for (int u = 0; u < U; ++u) a3[u] = b3[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < kQ; k0 += 32) {
          const FragBF bb = trfrag(sDY, LX, k0, ct * 16, li, lg);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            a3[u] = mma(trfrag(sMh, LQ, k0, (rt0 + u) * 16, li, lg), bb, a3[u]);
            a3[u] = mma(trfrag(sMl, LQ, k0, (rt0 + u) * 16, li, lg), bb, a3[u]);
          }
        }
#pragma unroll
        for (int k0 = 0; k0 < NP; k0 += 32) {
          const FragBF gh = kc16(sSh, LS, ct * 16 + li, k0, lg), gl = kc16(sSl, LS, ct * 16 + li, k0, lg);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const FragBF a = kc16(sB, LB, (rt0 + u) * 16 + li, k0, lg);
            b3[u] = mma(a, gh, b3[u]);
            b3[u] = mma(a, gl, b3[u]);
          }
        }
        const int pc = ct * 16 + li;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = (rt0 + u) * 16 + 4 * lg + r;
            const float br = a3[u][r] + sEout[t] * b3[u][r];
            if (t < nv && pc < P)
              p.dx[(((int64_t)b_ * L + t0 + t) * H + h) * P + pc] = Dh * (float)sDY[t * LX + pc] + sDel[t] * br;
            dp[u][r] += (float)sX[t * LX + pc] * br;
          }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = sum16(dp[u][r]);
          if (li == 0) dinP[ct0][(rt0 + u) * 16 + 4 * lg + r] = v;
        }
    }

    // --- X G: dB part e_out o (X G); v_j = e_out_j Delta_j sum_n B_jn (X G)_jn
    f32x4 acc6[U][NT / 2];
    {
      float vp[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) vp[u][r] = 0.f;
#pragma unroll
      for (int k = 0; k < NT / 2; ++k) {
        const int ct = ct0 + 2 * k;
        f32x4 acc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < PP; k0 += 32) {
          const FragBF th = trfrag(sSh, LS, k0, ct * 16, li, lg), tl = trfrag(sSl, LS, k0, ct * 16, li, lg);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const FragBF a = kc16(sX, LX, (rt0 + u) * 16 + li, k0, lg);
            acc[u] = mma(a, th, acc[u]);
            acc[u] = mma(a, tl, acc[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = (rt0 + u) * 16 + 4 * lg + r;
            vp[u][r] += (float)sB[t * LB + ct * 16 + li] * acc[u][r];
            acc6[u][k][r] = sEout[t] * acc[u][r];
          }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = sum16(vp[u][r]);
          if (li == 0) vP[ct0][(rt0 + u) * 16 + 4 * lg + r] = v;
        }
    }
    lds_barrier();
    uint4 nx[NPC], ndy[NPC];
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int piece = tid + i * NTH, xr_row = piece / XPC, xr_col = (piece % XPC) * 8;
      nx[i] = ndy[i] = make_uint4(0u, 0u, 0u, 0u);
      if (has_next && piece < NXP && xr_row < nv) {
        const int64_t off = (((int64_t)b_ * L + t0 + xr_row) * H + h + 1) * P + xr_col;
        nx[i] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const __bf16 *>(p.x) + off);
        ndy[i] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const __bf16 *>(p.dy) + off);
      }
    }

    // --- P2 = DX o E (split) to LDS; dB += Delta o (e_out o XG + P2^T C)
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          put_split(sMh, sMl, ((rt0 + u) * 16 + 4 * lg + r) * LQ + (ct0 + 2 * k) * 16 + li, P2[u][k][r]);
    lds_barrier();
#pragma unroll
    for (int k = 0; k < NT / 2; ++k) {
      const int ct = ct0 + 2 * k;
      f32x4 acc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u] = acc6[u][k];
#pragma unroll
      for (int k0 = 0; k0 < kQ; k0 += 32) {
        const FragBF bb = trfrag(sC, LB, k0, ct * 16, li, lg);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          acc[u] = mma(trfrag(sMh, LQ, k0, (rt0 + u) * 16, li, lg), bb, acc[u]);
          acc[u] = mma(trfrag(sMl, LQ, k0, (rt0 + u) * 16, li, lg), bb, acc[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) dBacc[u][k][r] += sDel[(rt0 + u) * 16 + 4 * lg + r] * acc[u][r];
    }

    // --- dC += P2 diag(Delta) B on the same planes: this wave's P2 rows
    //     as A fragments (hi + lo), each K-value (token j) scaled by Delta_j
    //     in registers and split again; no second pass through LDS
    FragBF ph[U][kQ / 32], pl[U][kQ / 32];
#pragma unroll
    for (int kk = 0; kk < kQ / 32; ++kk) {
      const float4 d0 = *reinterpret_cast<const float4 *>(&sDel[32 * kk + 4 * lg]);
      const float4 d1 = *reinterpret_cast<const float4 *>(&sDel[32 * kk + 16 + 4 * lg]);
      const float dj[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const FragBF h = kc16(sMh, LQ, (rt0 + u) * 16 + li, 32 * kk, lg);
        const FragBF l = kc16(sMl, LQ, (rt0 + u) * 16 + li, 32 * kk, lg);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = ((float)h.v[e] + (float)l.v[e]) * dj[e];
          ph[u][kk].v[e] = (__bf16)v;
          pl[u][kk].v[e] = (__bf16)(v - (float)ph[u][kk].v[e]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NT / 2; ++k) {
      const int ct = ct0 + 2 * k;
#pragma unroll
      for (int kk = 0; kk < kQ / 32; ++kk) {
        const FragBF bb = trfrag(sB, LB, 32 * kk, ct * 16, li, lg);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          dCacc[u][k] = mma(ph[u][kk], bb, dCacc[u][k]);
          dCacc[u][k] = mma(pl[u][kk], bb, dCacc[u][k]);
        }
      }
    }

    // --- da, ddt and the head's partial sums (wave 0, lane k = token); wave 1
    //     forms the next head's decays, waves 2.. split its entering state
    //     (in sGst) into the two planes and copy its G into sGst, piece by
    //     piece (each wave splits the pieces it then overwrites); every
    //     thread stores its x and dy pieces of the next head
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
      const int piece = tid + i * NTH, xr_row = piece / XPC, xr_col = (piece % XPC) * 8;
      if (has_next && piece < NXP) {
        *reinterpret_cast<uint4 *>(&sX[xr_row * LX + xr_col]) = nx[i];
        *reinterpret_cast<uint4 *>(&sDY[xr_row * LX + xr_col]) = ndy[i];
      }
    }
    if (w != 0) {
      if (has_next) {
        if (w == 1) {
          decay_of(h + 1, cur ^ 1);
        } else {
          __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
          const float *Gsrc = p.adj + (((int64_t)b_ * H + h + 1) * nc + c) * PN;
          const auto rsg = make_rsrc(Gsrc, (uint32_t)PN * 4u);
          for (int q = w - 2; q < PN / 256; q += NW - 2) {
            const int idx = q * 64 + lane; // float4 index
            const int r = (idx * 4) / N, col = (idx * 4) % N, off = r * LS + col;
            const float4 hv = *reinterpret_cast<const float4 *>(sGst + 4 * idx);
            const float hq[4] = {hv.x, hv.y, hv.z, hv.w};
            bf16x4 nh, nl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              nh[e] = (__bf16)hq[e];
              nl[e] = (__bf16)(hq[e] - (float)nh[e]);
            }
            *reinterpret_cast<bf16x4 *>(sSh + off) = nh;
            *reinterpret_cast<bf16x4 *>(sSl + off) = nl;
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rsg, (__attribute__((address_space(3))) void *)(sGst + q * 256), 16,
                                                     q * 1024 + lane * 16, 0, 0, 0);
          }
        }
      }
    } else {
      const int k = lane;
      const float colsum = colW[0][k] + colW[1][k] + colW[2][k] + colW[3][k];
      const float rowsum = rowW[0][k] + rowW[1][k];
      const float dlt = colsum - rowsum;
      const float R = wave_incl_scan(dlt) - dlt;
      const float uk = uP[0][k] + uP[1][k];
      const float u_incl = wave_incl_scan(uk);
      const float Uf = lane63(u_incl) - u_incl + uk;
      const float v = sEout[k] * sDel[k] * (vP[0][k] + vP[1][k]);
      const float V = wave_incl_scan(v) - v;
      float gh = 0.f;
#pragma unroll
      for (int q = 1; q <= NW; ++q) gh += sRed[q];
      const float da = R + Uf + V + hw_exp2(cum_last2) * gh;
      const float din = dinP[0][k] + dinP[1][k];
      const float ddt = (din + Ah * da) * sSig[k];
      const bool valid = k < nv;
      if (valid) p.ddt[((int64_t)b_ * L + t0 + k) * H + h] = ddt;
      const float pa = wave_sum(valid ? sDel[k] * da : 0.f);
      const float pd = wave_sum(valid ? sDiag[k] : 0.f);
      const float pb = wave_sum(valid ? ddt : 0.f);
      if (lane == 0) {
        float *q = p.part + (bh * nc + c) * 3;
        q[0] = pa;
        q[1] = pd;
        q[2] = pb;
      }
    }
    lds_barrier();
  }

#pragma unroll
  for (int u = 0; u < U; ++u)
#pragma unroll
    for (int k = 0; k < NT / 2; ++k) {
      const int n = (ct0 + 2 * k) * 16 + li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = (rt0 + u) * 16 + 4 * lg + r;
        if (t < nv && n < N) {
          const int64_t o = (((int64_t)b_ * L + t0 + t) * G + g) * N + n;
          p.dB[o] = dBacc[u][k][r];
          p.dC[o] = dCacc[u][k][r];
        }
      }
    }
}

template <int P, int N>
__global__ void __launch_bounds__(512) bwd_chunk_bf16_kernel(const BwdParams p) {
  chunk_bf16_body<P, N, 8>(p);
}

// Gradient through the output gate out = y * silu(z): dy = dout * silu(z)
// (stored in the input dtype, the backward's dout) and
// dz = dout * y * silu'(z) with silu'(z) = s + z s (1 - s), s the logistic.
// Four elements per thread (the element count is a multiple of 16).
template <typename T> __device__ __forceinline__ void ld4(const T *p, float *v);
template <> __device__ __forceinline__ void ld4<__bf16>(const __bf16 *p, float *v) {
  const bf16x4 a = *reinterpret_cast<const bf16x4 *>(p);
  v[0] = (float)a[0]; v[1] = (float)a[1]; v[2] = (float)a[2]; v[3] = (float)a[3];
}
template <> __device__ __forceinline__ void ld4<float>(const float *p, float *v) {
  const float4 a = *reinterpret_cast<const float4 *>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
template <typename T>
__global__ void __launch_bounds__(256) gate_bwd_kernel(const T *__restrict__ y, const T *__restrict__ z,
                                                       const T *__restrict__ dout, T *__restrict__ dy,
                                                       float *__restrict__ dz, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  float yv[4], zv[4], gv[4], a[4], b[4];
  ld4<T>(y + 4 * i, yv);
  ld4<T>(z + 4 * i, zv);
  ld4<T>(dout + 4 * i, gv);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float sg = __builtin_amdgcn_rcpf(1.f + hw_exp2(-zv[k] * kLog2e));
    a[k] = gv[k] * zv[k] * sg;
    b[k] = gv[k] * yv[k] * (sg + zv[k] * sg * (1.f - sg));
  }
  st4<T>(dy + 4 * i, a[0], a[1], a[2], a[3]);
  *reinterpret_cast<float4 *>(dz + 4 * i) = make_float4(b[0], b[1], b[2], b[3]);
}

// With several segments per walk (each walked from zero): add the carried-in
// state of each chunk's segment (after the fold over segments, which starts
// from init / dfinal), decayed to the chunk boundary: states[c] += 2^fpre[c]
// C_s, adj[c] += 2^rpre[c] C'_s (C'_s in fold slot nseg-1-s), and the
// gradient of the initial state dinit += 2^rdec0 C'_0.  One float4 per thread.
__global__ void __launch_bounds__(256) bwd_fixup_kernel(const BwdParams p, int PN) {
  const int64_t nbh = (int64_t)p.b * p.H, per = (int64_t)p.nc * (PN / 4);
  const int64_t n1 = nbh * per, id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int nseg = p.nseg, cps = p.seg_chunks, PN4 = PN / 4;
  if (id < 2 * n1) {
    const bool rev = id >= n1;
    const int64_t j = rev ? id - n1 : id;
    const int64_t bh = j / per;
    const int c = (int)((j % per) / PN4), e4 = (int)(j % PN4);
    const int sgm = c / cps;
    const int slot = rev ? nseg - 1 - sgm : sgm;
    const float f = hw_exp2((rev ? p.rpre : p.fpre)[bh * p.nc + c]);
    const float4 cv = reinterpret_cast<const float4 *>((rev ? p.segend_r : p.segend_f) + (bh * nseg + slot) * PN)[e4];
    float4 *d = reinterpret_cast<float4 *>((rev ? p.adj : p.states) + (bh * p.nc + c) * PN) + e4;
    float4 v = *d;
    v.x += f * cv.x; v.y += f * cv.y; v.z += f * cv.z; v.w += f * cv.w;
    *d = v;
  } else if (p.dinit && id < 2 * n1 + nbh * PN4) {
    const int64_t j = id - 2 * n1, bh = j / PN4;
    const int e4 = (int)(j % PN4);
    const float f = hw_exp2(p.rdec0[bh]);
    const float4 cv = reinterpret_cast<const float4 *>(p.segend_r + (bh * nseg + nseg - 1) * PN)[e4];
    float4 *d = reinterpret_cast<float4 *>(p.dinit + bh * PN) + e4;
    float4 v = *d;
    v.x += f * cv.x; v.y += f * cv.y; v.z += f * cv.z; v.w += f * cv.w;
    *d = v;
  }
}

// dA, dD, d dt_bias per head: one workgroup per head sums the (batch, chunk)
// partials, each thread a fixed strided subset, then a fixed shuffle tree and
// a fixed order over the four waves, so the result is the same every run.
__global__ void __launch_bounds__(256) bwd_param_kernel(const float *__restrict__ part, float *__restrict__ dA,
                                                        float *__restrict__ dD, float *__restrict__ ddt_bias,
                                                        int b, int H, int nc) {
  __shared__ float red[3][4];
  const int h = blockIdx.x, tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  float sa = 0.f, sd = 0.f, sb = 0.f;
  for (int k = tid; k < b * nc; k += 256) {
    const int ib = k / nc, c = k % nc;
    const float *q = part + (((int64_t)ib * H + h) * nc + c) * 3;
    sa += q[0];
    sd += q[1];
    sb += q[2];
  }
  sa = wave_sum(sa);
  sd = wave_sum(sd);
  sb = wave_sum(sb);
  if (lane == 0) {
    red[0][w] = sa;
    red[1][w] = sd;
    red[2][w] = sb;
  }
  __syncthreads();
  if (tid == 0) {
    dA[h] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    if (dD) dD[h] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    if (ddt_bias) ddt_bias[h] = (red[2][0] + red[2][1]) + (red[2][2] + red[2][3]);
  }
}

template <typename T, int P, int N> hipError_t launch_bwd_t(const BwdParams &p, hipStream_t st) {
  // the forward and the backward state walks (and their segments), together in one launch
  const dim3 grid_bh((unsigned)(2 * p.b * p.H * p.nseg));
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((bwd_state_scan_bf16_kernel<P, N>), grid_bh, dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_state_scan_kernel<T, P, N>), grid_bh, dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.nseg > 1) {
    // fold the segment end states in order (reverse ones stored reversed),
    // then add each segment's carried-in state into its chunks
    e = launch_state_pass(p.segend_f, p.segdec_f, p.states_init, p.b, p.H, P * N, p.nseg, st);
    if (e != hipSuccess) return e;
    e = launch_state_pass(p.segend_r, p.segdec_r, p.dfinal, p.b, p.H, P * N, p.nseg, st);
    if (e != hipSuccess) return e;
    const int64_t n = 2 * (int64_t)p.b * p.H * p.nc * (P * N / 4) + (int64_t)p.b * p.H * (P * N / 4);
    hipLaunchKernelGGL(bwd_fixup_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, P * N);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((bwd_chunk_bf16_kernel<P, N>), dim3((unsigned)(p.b * p.G * p.nc)), dim3(512), 0, st, p);
  else
    hipLaunchKernelGGL((bwd_chunk_kernel<T, P, N>), dim3((unsigned)(p.b * p.G * p.nc)), dim3(512), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_param_kernel, dim3((unsigned)p.H), dim3(256), 0, st, p.part, p.dA, p.dD, p.ddt_bias,
                     p.b, p.H, p.nc);
  return hipGetLastError();
}

template <typename T, int P> hipError_t launch_bwd_n(int N, const BwdParams &p, hipStream_t st) {
  switch (N) {
  case 16: return launch_bwd_t<T, P, 16>(p, st);
  case 32: return launch_bwd_t<T, P, 32>(p, st);
  case 64: return launch_bwd_t<T, P, 64>(p, st);
  case 128: return launch_bwd_t<T, P, 128>(p, st);
  }
  return hipErrorInvalidValue;
}
template <typename T> hipError_t launch_bwd_p(int P, int N, const BwdParams &p, hipStream_t st) {
  switch (P) {
  case 16: return launch_bwd_n<T, 16>(N, p, st);
  case 32: return launch_bwd_n<T, 32>(N, p, st);
  case 64: return launch_bwd_n<T, 64>(N, p, st);
  }
  return hipErrorInvalidValue;
}

} // namespace

hipError_t launch_gate_bwd(int dtype, const void *y, const void *z, const void *dout, void *dy, float *dz,
                           int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  const dim3 grid((unsigned)((n4 + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(gate_bwd_kernel<__bf16>, grid, dim3(256), 0, st, (const __bf16 *)y, (const __bf16 *)z,
                       (const __bf16 *)dout, (__bf16 *)dy, dz, n4);
  else
    hipLaunchKernelGGL(gate_bwd_kernel<float>, grid, dim3(256), 0, st, (const float *)y, (const float *)z,
                       (const float *)dout, (float *)dy, dz, n4);
  return hipGetLastError();
}

hipError_t launch_bwd(int dtype, int P, int N, const BwdParams &p, hipStream_t st) {
  return dtype == 1 ? launch_bwd_p<__bf16>(P, N, p, st) : launch_bwd_p<float>(P, N, p, st);
}

} // namespace ssd
