// ssd_kernels.hip -- gfx950 kernels of the Mamba-2 SSD scan.
//
// The method ("Mamba-3 deep dive ch. 2, SSM foundations", 171host.com):
//   section 2.1.2  h_t = alpha_t h_{t-1} + Delta_t B_t x_t,
//                  alpha_t = exp(Delta_t A), y_t = C_t^T h_t
//   section 2.2.1  the same map as one matrix product Y = (L o C B^T) X whose
//                  mask entry L_ij is the product of the forget gates after j
//                  up to i (1 on the diagonal, 0 above it)
// plus D x from the output equation of section 2.1.1, and
// Delta = softplus(dt + dt_bias) (Mamba reading notes, sxlin0.github.io,
// selective mechanism).  "Transformers are SSMs" summary
// (gongshangzheng.github.io), sections 1.1-1.2: off-diagonal blocks of the
// mask have rank <= N, so a long sequence is cut into blocks, each block
// evaluated with the quadratic form and the blocks linked through the
// N-dimensional state.
//
// Block algebra used below, for a block starting after state S (P x N),
// with cum_i the inclusive sum of Delta*A over the block up to token i:
//   y_i   = exp(cum_i) S C_i                                     (state term)
//         + sum_{j<=i} exp(cum_i - cum_j) (C_i . B_j) Delta_j x_j  (intra)
//         + D x_i
//   S'    = exp(cum_last) S + sum_j exp(cum_last - cum_j) Delta_j x_j B_j^T
//
// One workgroup walks its (batch, head, segment) in 64-token sub-blocks
// with the P x N state held in MFMA accumulator registers.  Wave w owns
// state rows p in [16w, 16w+16).  Per sub-block:
//   S^T tile  = B C^T            (MFMA, K = N)         -> masked, scaled M
//   Y^T       = exp(cum) (S C^T) (MFMA, K = N, A operand = state registers)
//             + X^T M^T          (MFMA, K = tokens)
//   S^T'      = decay * S^T + (B^T) (w o X)  (MFMA, K = tokens)
// All contractions use v_mfma_f32_16x16x32_bf16 (bf16 inputs) or eight
// v_mfma_f32_16x16x4f32 (fp32 inputs) with fp32 accumulation.
//
// Fragment convention for a 16x16 tile and one K-step of 32: lane l supplies
// row/column (l % 16) and eight K-values selected by the lane group l / 16;
// the A and B operands use the same K selection, so the K order inside a
// step is free.  The accumulator holds D[4*(l/16) + r][l % 16], r = 0..3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_internal.h"

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct FragBF {
  bf16x8 v;
};
struct FragF32 {
  float v[8];
};
template <typename T> struct FragOf;
template <> struct FragOf<__bf16> { using type = FragBF; };
template <> struct FragOf<float> { using type = FragF32; };

__device__ __forceinline__ f32x4 mma(const FragBF &a, const FragBF &b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(const FragF32 &a, const FragF32 &b, f32x4 c) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], c, 0, 0, 0);
  return c;
}

// 8 consecutive elements (16 B for bf16, 32 B for fp32) from LDS.
__device__ __forceinline__ FragBF ld8(const __bf16 *p) {
  FragBF f;
  f.v = *reinterpret_cast<const bf16x8 *>(p);
  return f;
}
__device__ __forceinline__ FragF32 ld8(const float *p) {
  FragF32 f;
  float4 a = *reinterpret_cast<const float4 *>(p);
  float4 b = *reinterpret_cast<const float4 *>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}
// 4 consecutive elements at p0 then 4 at p1.
__device__ __forceinline__ FragBF ld4x2(const __bf16 *p0, const __bf16 *p1) {
  bf16x4 a = *reinterpret_cast<const bf16x4 *>(p0);
  bf16x4 b = *reinterpret_cast<const bf16x4 *>(p1);
  FragBF f;
  f.v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ FragF32 ld4x2(const float *p0, const float *p1) {
  FragF32 f;
  float4 a = *reinterpret_cast<const float4 *>(p0);
  float4 b = *reinterpret_cast<const float4 *>(p1);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}

template <typename T> __device__ __forceinline__ typename FragOf<T>::type pack8(const float *v);
template <> __device__ __forceinline__ FragBF pack8<__bf16>(const float *v) {
  FragBF f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (__bf16)v[e];
  return f;
}
template <> __device__ __forceinline__ FragF32 pack8<float>(const float *v) {
  FragF32 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = v[e];
  return f;
}

template <typename T> __device__ __forceinline__ void st4(T *p, float a, float b, float c, float d);
template <> __device__ __forceinline__ void st4<__bf16>(__bf16 *p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4 *>(p) = v;
}
template <> __device__ __forceinline__ void st4<float>(float *p, float a, float b, float c, float d) {
  *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

__device__ __forceinline__ float to_f(__bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f(float v) { return v; }

// softplus(z) = log(1 + e^z) = max(z, 0) + log1p(e^{-|z|}).
__device__ __forceinline__ float softplus_f(float z) {
  return fmaxf(z, 0.f) + log1pf(__expf(-fabsf(z)));
}

// ---------------------------------------------------------------------------
// The chunk walk.
template <typename T, int P, int N, int MODE>
__global__ void __launch_bounds__(P / 16 * 64)
walk_kernel(const WalkParams prm) {
  constexpr bool kOut = MODE != kWalkChunkState;
  constexpr int NW = P / 16;             // waves; wave w owns rows [16w, 16w+16)
  constexpr int NTH = NW * 64;
  constexpr int NP = (N + 31) / 32 * 32; // N padded to a K-step
  constexpr int NTILE = NP / 16;
  constexpr int KN = NP / 32;
  constexpr int VEC = 16 / (int)sizeof(T); // elements per 16-byte access
  constexpr int LDB = NP + VEC;            // row stride of the [token][n] tiles
  constexpr int LDJ = kSub + VEC;          // row stride of the [.][token] tiles
  constexpr int NTI = kSub / 16;           // token tiles per sub-block

  __shared__ __attribute__((aligned(16))) T sB[kOut ? kSub * LDB : VEC];
  __shared__ __attribute__((aligned(16))) T sC[kOut ? kSub * LDB : VEC];
  __shared__ __attribute__((aligned(16))) T sBt[NP * LDJ];
  __shared__ __attribute__((aligned(16))) T sXt[P * LDJ];
  __shared__ __attribute__((aligned(16))) T sM[kOut ? kSub * LDJ : VEC];
  __shared__ float sCum[kSub];
  __shared__ float sDel[kSub];

  const int H = prm.H, G = prm.G, L = prm.L, nseg = prm.nseg;
  const int W = prm.b * H * nseg;
  // XCD-aware order: consecutive workgroup ids are dealt round-robin to the
  // 8 XCDs, so give each XCD a contiguous range of (batch, segment, head)
  // ids; heads of one (batch, segment) then share B/C through one L2.
  const int bid = blockIdx.x;
  const int logical = (W % 8 == 0) ? (bid % 8) * (W / 8) + bid / 8 : bid;
  const int h = logical % H;
  const int seg = (logical / H) % nseg;
  const int ib = logical / (H * nseg);
  const int g = (int)((int64_t)h * G / H);
  const int t_begin = seg * prm.seg_len;
  const int t_end = min(L, t_begin + prm.seg_len);

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int prow = 16 * w + lr; // the state row this lane feeds as an operand

  const T *__restrict__ xg = reinterpret_cast<const T *>(prm.x);
  const T *__restrict__ Bg = reinterpret_cast<const T *>(prm.B);
  const T *__restrict__ Cg = reinterpret_cast<const T *>(prm.C);
  const float a_h = prm.A[h];
  const float d_h = prm.D ? prm.D[h] : 0.f;
  const float bias = (MODE == kWalkFull && prm.dt_bias) ? prm.dt_bias[h] : 0.f;
  const int64_t state_idx = ((int64_t)(ib * H + h) * nseg + seg) * P * N;

  // State S^T tiles: hs[nt][r] = S[p = prow][n = 16 nt + 4 lg + r].
  f32x4 hs[NTILE];
#pragma unroll
  for (int nt = 0; nt < NTILE; ++nt) {
    const int n0 = 16 * nt + 4 * lg;
    if (prm.init && n0 < N)
      hs[nt] = *reinterpret_cast<const f32x4 *>(prm.init + state_idx + (int64_t)prow * N + n0);
    else
      hs[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int t0 = t_begin; t0 < t_end; t0 += kSub) {
    const int nv = min(kSub, t_end - t0);
    __syncthreads(); // previous sub-block is done with LDS

    // ---- stage B (and B^T), C and X^T of this sub-block into LDS ----------
    for (int idx = tid; idx < kSub * (NP / VEC); idx += NTH) {
      const int j = idx / (NP / VEC), n0 = (idx % (NP / VEC)) * VEC;
      float4 vb = make_float4(0.f, 0.f, 0.f, 0.f), vc = vb;
      if (j < nv && n0 < N) {
        const int64_t off = ((int64_t)(ib * L + t0 + j) * G + g) * N + n0;
        vb = *reinterpret_cast<const float4 *>(Bg + off);
        if (kOut) vc = *reinterpret_cast<const float4 *>(Cg + off);
      }
      if (kOut) {
        *reinterpret_cast<float4 *>(&sB[j * LDB + n0]) = vb;
        *reinterpret_cast<float4 *>(&sC[j * LDB + n0]) = vc;
      }
      const T *e = reinterpret_cast<const T *>(&vb);
#pragma unroll
      for (int q = 0; q < VEC; ++q) sBt[(n0 + q) * LDJ + j] = e[q];
    }
    for (int idx = tid; idx < kSub * (P / VEC); idx += NTH) {
      const int j = idx / (P / VEC), p0 = (idx % (P / VEC)) * VEC;
      float4 vx = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < nv) vx = *reinterpret_cast<const float4 *>(xg + ((int64_t)(ib * L + t0 + j) * H + h) * P + p0);
      const T *e = reinterpret_cast<const T *>(&vx);
#pragma unroll
      for (int q = 0; q < VEC; ++q) sXt[(p0 + q) * LDJ + j] = e[q];
    }
    if (w == 0) {
      // Delta and the inclusive cumsum of Delta*A over the sub-block (wave
      // scan, lane = token).  Padding tokens get Delta = 0: no decay, no
      // contribution.
      float dl = 0.f;
      if (l < nv) {
        if (MODE == kWalkFull)
          dl = softplus_f(prm.dt[(int64_t)(ib * L + t0 + l) * H + h] + bias);
        else
          dl = prm.dt[(int64_t)(ib * H + h) * L + t0 + l];
      }
      float cum = dl * a_h;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float v = __shfl_up(cum, off, 64);
        if (l >= off) cum += v;
      }
      sCum[l] = cum;
      sDel[l] = dl;
    }
    __syncthreads();

    f32x4 yacc[NTI];
    if constexpr (kOut) {
      // ---- masked scores M[i][j] = (C_i . B_j) exp(cum_i - cum_j) Delta_j --
      // Tiles (jt, it) with jt <= it, plus the all-zero tile above the
      // diagonal that the K-step of 32 tokens reads for even it.
      constexpr int NMT = NTI * (NTI + 1) / 2 + NTI / 2;
      for (int tile = w; tile < NMT; tile += NW) {
        int it = 0, rem = tile;
        while (rem >= it + 1 + ((it & 1) == 0 ? 1 : 0)) {
          rem -= it + 1 + ((it & 1) == 0 ? 1 : 0);
          ++it;
        }
        const int jt = rem;
        const int i = 16 * it + lr;
        float m[4] = {0.f, 0.f, 0.f, 0.f};
        if (jt <= it) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KN; ++ks)
            acc = mma(ld8(&sB[(16 * jt + lr) * LDB + 32 * ks + 8 * lg]),
                      ld8(&sC[i * LDB + 32 * ks + 8 * lg]), acc);
          const float ci = sCum[i];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * jt + 4 * lg + r;
            m[r] = (j <= i) ? acc[r] * __expf(ci - sCum[j]) * sDel[j] : 0.f;
          }
        }
        st4<T>(&sM[i * LDJ + 16 * jt + 4 * lg], m[0], m[1], m[2], m[3]);
      }

      // ---- state term: Y^T[p][i] = exp(cum_i) sum_n S[p][n] C[i][n] --------
      typename FragOf<T>::type hf[KN];
#pragma unroll
      for (int ks = 0; ks < KN; ++ks) {
        float v[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[r] = hs[2 * ks][r];
          v[4 + r] = hs[2 * ks + 1][r];
        }
        hf[ks] = pack8<T>(v);
      }
#pragma unroll
      for (int it = 0; it < NTI; ++it) {
        const int i = 16 * it + lr;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KN; ++ks)
          acc = mma(hf[ks],
                    ld4x2(&sC[i * LDB + 32 * ks + 4 * lg], &sC[i * LDB + 32 * ks + 16 + 4 * lg]),
                    acc);
        const float e = __expf(sCum[i]);
        yacc[it] = acc * e;
      }
    }
    __syncthreads(); // M complete

    if constexpr (kOut) {
      // ---- intra-block term: Y^T[p][i] += sum_{j<=i} X^T[p][j] M[i][j] -----
#pragma unroll
      for (int it = 0; it < NTI; ++it) {
#pragma unroll
        for (int ks = 0; ks < (16 * (it + 1) + 31) / 32; ++ks)
          yacc[it] = mma(ld8(&sXt[prow * LDJ + 32 * ks + 8 * lg]),
                         ld8(&sM[(16 * it + lr) * LDJ + 32 * ks + 8 * lg]), yacc[it]);
      }
      // ---- epilogue: + D x, store y --------------------------------------
      T *__restrict__ og = reinterpret_cast<T *>(prm.out);
#pragma unroll
      for (int it = 0; it < NTI; ++it) {
        const int i = 16 * it + lr;
        if (i < nv) {
          const int p0 = 16 * w + 4 * lg;
          float y[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = yacc[it][r] + d_h * to_f(sXt[(p0 + r) * LDJ + i]);
          st4<T>(og + ((int64_t)(ib * L + t0 + i) * H + h) * P + p0, y[0], y[1], y[2], y[3]);
        }
      }
    }

    // ---- state update: S^T = decay S^T + B^T (w o X), w_j = e^{cum_last-cum_j} Delta_j
    const float clast = sCum[kSub - 1];
    const float dec = __expf(clast);
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) hs[nt] *= dec;
#pragma unroll
    for (int ks = 0; ks < kSub / 32; ++ks) {
      float v[8];
      const T *xp = &sXt[prow * LDJ + 32 * ks + 8 * lg];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 32 * ks + 8 * lg + e;
        v[e] = to_f(xp[e]) * (__expf(clast - sCum[j]) * sDel[j]);
      }
      const auto bx = pack8<T>(v);
#pragma unroll
      for (int nt = 0; nt < NTILE; ++nt)
        hs[nt] = mma(ld8(&sBt[(16 * nt + lr) * LDJ + 32 * ks + 8 * lg]), bx, hs[nt]);
    }
  }

  if (prm.state_out) {
#pragma unroll
    for (int nt = 0; nt < NTILE; ++nt) {
      const int n0 = 16 * nt + 4 * lg;
      if (n0 < N)
        *reinterpret_cast<f32x4 *>(prm.state_out + state_idx + (int64_t)prow * N + n0) = hs[nt];
    }
  }
}

// ---------------------------------------------------------------------------
// Per-chunk log-decay: Delta = softplus(dt + bias) and the chunk-local
// inclusive cumsum of Delta * A.  One thread per (batch, chunk, head);
// consecutive threads are consecutive heads, so the dt reads coalesce.
__global__ void __launch_bounds__(256)
cumsum_kernel(const float *__restrict__ dt, const float *__restrict__ dt_bias,
              const float *__restrict__ A, float *__restrict__ delta,
              float *__restrict__ cum, int b, int L, int H, int chunk) {
  const int nc = (L + chunk - 1) / chunk;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (int64_t)b * nc * H) return;
  const int h = (int)(id % H);
  const int c = (int)((id / H) % nc);
  const int ib = (int)(id / ((int64_t)H * nc));
  const float bias = dt_bias ? dt_bias[h] : 0.f;
  const float a = A[h];
  const int t_end = min(L, (c + 1) * chunk);
  float run = 0.f;
  for (int t = c * chunk; t < t_end; ++t) {
    const float d = softplus_f(dt[((int64_t)ib * L + t) * H + h] + bias);
    run += d * a;
    delta[((int64_t)ib * H + h) * L + t] = d;
    cum[((int64_t)ib * H + h) * L + t] = run;
  }
}

// ---------------------------------------------------------------------------
// Inter-chunk state passing, sequential over chunks and parallel over
// (batch, head, P*N/4): each thread carries four consecutive fp32 state
// entries.  Slot c of `states` holds chunk c's own (zero-entry) end state on
// input and the state entering chunk c on output.  The chunk decays
// exp(cum at the chunk's last token) are read by lane c of a wave and
// broadcast with wave shuffles.
__global__ void __launch_bounds__(256)
state_pass_kernel(float *__restrict__ states, const float *__restrict__ cum,
                  const float *__restrict__ init, float *__restrict__ final_state,
                  int b, int L, int H, int PN, int chunk) {
  const int nc = (L + chunk - 1) / chunk;
  const int per_bh = PN / 4;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t bh = id / per_bh;
  const int e4 = (int)(id % per_bh);
  const bool live = bh < (int64_t)b * H;
  const int lane = threadIdx.x & 63;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live && init) s = reinterpret_cast<const float4 *>(init + bh * PN)[e4];
  float4 *base = reinterpret_cast<float4 *>(states + (live ? bh : 0) * (int64_t)nc * PN) + e4;
  const float *cb = cum + (live ? bh : 0) * (int64_t)L;
  for (int c0 = 0; c0 < nc; c0 += 64) {
    // lane k holds the decay of chunk c0 + k
    float my_dec = 1.f;
    if (c0 + lane < nc) my_dec = __expf(cb[min(L, (c0 + lane + 1) * chunk) - 1]);
    const int cnt = min(64, nc - c0);
    int k = 0;
    for (; k + 4 <= cnt; k += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = live ? base[(int64_t)(c0 + k + u) * per_bh] : make_float4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float d = __shfl(my_dec, k + u, 64);
        if (live) base[(int64_t)(c0 + k + u) * per_bh] = s;
        s.x = d * s.x + v[u].x; s.y = d * s.y + v[u].y;
        s.z = d * s.z + v[u].z; s.w = d * s.w + v[u].w;
      }
    }
    for (; k < cnt; ++k) {
      const float4 v = live ? base[(int64_t)(c0 + k) * per_bh] : make_float4(0, 0, 0, 0);
      const float d = __shfl(my_dec, k, 64);
      if (live) base[(int64_t)(c0 + k) * per_bh] = s;
      s.x = d * s.x + v.x; s.y = d * s.y + v.y;
      s.z = d * s.z + v.z; s.w = d * s.w + v.w;
    }
  }
  if (live && final_state) reinterpret_cast<float4 *>(final_state + bh * PN)[e4] = s;
}

// ---------------------------------------------------------------------------
// Recurrent step ("From Transformer to Mamba", section 2.1, single-step
// update): one workgroup per (batch, head); N/4 threads per state row, each
// owning four consecutive entries; the readout sum over n is a shuffle
// reduction inside those N/4 lanes.
template <typename T, int N>
__global__ void __launch_bounds__(256)
step_kernel(float *__restrict__ state, const T *__restrict__ x,
            const float *__restrict__ dt, const float *__restrict__ A,
            const T *__restrict__ B, const T *__restrict__ C,
            const float *__restrict__ D, T *__restrict__ out, int H, int P, int G) {
  constexpr int TPR = N / 4;       // threads per row
  constexpr int RPP = 256 / TPR;   // rows per pass
  constexpr int BATCH = 8;         // passes whose loads are issued together
  const int bh = blockIdx.x;
  const int ib = bh / H, h = bh % H;
  const int g = (int)((int64_t)h * G / H);
  const int tid = threadIdx.x;
  const int rp = tid / TPR, c4 = tid % TPR;
  const float dl = dt[bh];
  const float alpha = __expf(dl * A[h]);
  const float d_h = D ? D[h] : 0.f;
  float bv[4], cv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    bv[q] = to_f(B[((int64_t)ib * G + g) * N + 4 * c4 + q]);
    cv[q] = to_f(C[((int64_t)ib * G + g) * N + 4 * c4 + q]);
  }
  float4 *srow = reinterpret_cast<float4 *>(state + (int64_t)bh * P * N);
  for (int p0 = 0; p0 < P; p0 += RPP * BATCH) {
    float4 s[BATCH];
    float xv[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int p = p0 + u * RPP + rp;
      if (p < P) {
        s[u] = srow[(int64_t)p * TPR + c4];
        xv[u] = to_f(x[(int64_t)bh * P + p]);
      } else {
        s[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        xv[u] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int p = p0 + u * RPP + rp;
      const float in = dl * xv[u];
      s[u].x = alpha * s[u].x + in * bv[0];
      s[u].y = alpha * s[u].y + in * bv[1];
      s[u].z = alpha * s[u].z + in * bv[2];
      s[u].w = alpha * s[u].w + in * bv[3];
      float acc = s[u].x * cv[0] + s[u].y * cv[1] + s[u].z * cv[2] + s[u].w * cv[3];
#pragma unroll
      for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if (p < P) {
        srow[(int64_t)p * TPR + c4] = s[u];
        if (c4 == 0) out[(int64_t)bh * P + p] = (T)(acc + d_h * xv[u]);
      }
    }
  }
}

template <typename T, int P, int N>
hipError_t launch_walk_t(WalkMode mode, const WalkParams &p, hipStream_t st) {
  const dim3 grid((unsigned)(p.b * p.H * p.nseg)), block(P / 16 * 64);
  switch (mode) {
  case kWalkFull: hipLaunchKernelGGL((walk_kernel<T, P, N, kWalkFull>), grid, block, 0, st, p); break;
  case kWalkChunkOut: hipLaunchKernelGGL((walk_kernel<T, P, N, kWalkChunkOut>), grid, block, 0, st, p); break;
  case kWalkChunkState: hipLaunchKernelGGL((walk_kernel<T, P, N, kWalkChunkState>), grid, block, 0, st, p); break;
  }
  return hipGetLastError();
}

template <typename T, int P>
hipError_t launch_walk_n(int N, WalkMode mode, const WalkParams &p, hipStream_t st) {
  switch (N) {
  case 16: return launch_walk_t<T, P, 16>(mode, p, st);
  case 32: return launch_walk_t<T, P, 32>(mode, p, st);
  case 64: return launch_walk_t<T, P, 64>(mode, p, st);
  case 128: return launch_walk_t<T, P, 128>(mode, p, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_walk_p(int P, int N, WalkMode mode, const WalkParams &p, hipStream_t st) {
  switch (P) {
  case 16: return launch_walk_n<T, 16>(N, mode, p, st);
  case 32: return launch_walk_n<T, 32>(N, mode, p, st);
  case 64: return launch_walk_n<T, 64>(N, mode, p, st);
  case 128: return launch_walk_n<T, 128>(N, mode, p, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_step_t(int N, float *state, const void *x, const float *dt, const float *A,
                         const void *B, const void *C, const float *D, void *out, int b,
                         int H, int P, int G, hipStream_t st) {
  const dim3 grid((unsigned)(b * H)), block(256);
  const T *xx = (const T *)x, *BB = (const T *)B, *CC = (const T *)C;
  T *oo = (T *)out;
  switch (N) {
  case 16: hipLaunchKernelGGL((step_kernel<T, 16>), grid, block, 0, st, state, xx, dt, A, BB, CC, D, oo, H, P, G); break;
  case 32: hipLaunchKernelGGL((step_kernel<T, 32>), grid, block, 0, st, state, xx, dt, A, BB, CC, D, oo, H, P, G); break;
  case 64: hipLaunchKernelGGL((step_kernel<T, 64>), grid, block, 0, st, state, xx, dt, A, BB, CC, D, oo, H, P, G); break;
  case 128: hipLaunchKernelGGL((step_kernel<T, 128>), grid, block, 0, st, state, xx, dt, A, BB, CC, D, oo, H, P, G); break;
  case 256: hipLaunchKernelGGL((step_kernel<T, 256>), grid, block, 0, st, state, xx, dt, A, BB, CC, D, oo, H, P, G); break;
  default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

} // namespace

hipError_t launch_walk(int dtype, int P, int N, WalkMode mode, const WalkParams &p,
                       hipStream_t stream) {
  return dtype == 1 ? launch_walk_p<__bf16>(P, N, mode, p, stream)
                    : launch_walk_p<float>(P, N, mode, p, stream);
}

hipError_t launch_cumsum(const float *dt, const float *dt_bias, const float *A, float *delta,
                         float *cum, int b, int L, int H, int chunk, hipStream_t stream) {
  const int nc = (L + chunk - 1) / chunk;
  const int64_t n = (int64_t)b * nc * H;
  hipLaunchKernelGGL(cumsum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dt,
                     dt_bias, A, delta, cum, b, L, H, chunk);
  return hipGetLastError();
}

hipError_t launch_state_pass(float *states, const float *cum, const float *init,
                             float *final_state, int b, int L, int H, int PN, int chunk,
                             hipStream_t stream) {
  const int64_t n = (int64_t)b * H * (PN / 4);
  hipLaunchKernelGGL(state_pass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     states, cum, init, final_state, b, L, H, PN, chunk);
  return hipGetLastError();
}

hipError_t launch_step(int dtype, int N, float *state, const void *x, const float *dt,
                       const float *A, const void *B, const void *C, const float *D, void *out,
                       int b, int H, int P, int G, hipStream_t stream) {
  return dtype == 1 ? launch_step_t<__bf16>(N, state, x, dt, A, B, C, D, out, b, H, P, G, stream)
                    : launch_step_t<float>(N, state, x, dt, A, B, C, D, out, b, H, P, G, stream);
}

} // namespace ssd
