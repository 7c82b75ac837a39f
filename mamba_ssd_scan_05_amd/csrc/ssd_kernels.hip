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

#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

// Masked-score tiles of a 64-token sub-block, enumerated row-tile major:
// (it, jt) with jt <= it, plus the all-zero tile (it, it+1) for even it that
// the 32-token K-steps of the intra-block product read.  Slots:
// (0,0) (0,1z) (1,0) (1,1) (2,0) (2,1) (2,2) (2,3z) (3,0) (3,1) (3,2) (3,3)
__host__ __device__ constexpr int mtile_it(int slot) { return slot < 4 ? slot / 2 : 2 + (slot - 4) / 4; }
__host__ __device__ constexpr int mtile_jt(int slot) {
  return slot - (mtile_it(slot) < 2 ? 2 * mtile_it(slot) : 4 * mtile_it(slot) - 4);
}

// ---------------------------------------------------------------------------
// The chunk walk.
//
// Work split inside a workgroup: KH * P/16 waves (KH = 1 or 2).  Wave w
// handles p-tile pt = w % (P/16) (state rows [16pt, 16pt+16)) and part
// hv = w / (P/16) of KH: it owns the n-tiles [hv*NTILE/KH, (hv+1)*NTILE/KH)
// of those state rows in registers and the output token tiles
// [hv*4/KH, (hv+1)*4/KH) of each sub-block.  With KH = 2 the operand copy
// of the whole state, which the state term needs, is exchanged through LDS
// once per sub-block; with KH = 1 it comes straight from the registers.
template <typename T, int P>
constexpr int walk_halves() { return 1; }
template <typename T, int P>
constexpr int walk_waves() { return walk_halves<T, P>() * (P / 16); }
template <typename T, int P>
constexpr int walk_min_waves_per_eu() {
  return (sizeof(T) == 2 && P == 64) ? (walk_halves<T, P>() == 2 ? 4 : 2) : 1;
}

template <typename T, int P, int N, int MODE>
__global__ void __launch_bounds__((walk_waves<T, P>() * 64), (walk_min_waves_per_eu<T, P>()))
walk_kernel(const WalkParams prm) {
  static_assert(kSub == 64, "the tile tables assume 64-token sub-blocks");
  constexpr bool kOut = MODE != kWalkChunkState;
  constexpr int NPT = P / 16;            // p-tiles
  constexpr int KH = walk_halves<T, P>();
  constexpr int NW = walk_waves<T, P>(); // waves
  constexpr int NTH = NW * 64;
  constexpr int NP = (N + 31) / 32 * 32; // N padded to a K-step
  constexpr int NTILE = NP / 16;
  constexpr int NTH2 = NTILE / KH;       // n-tiles per wave
  constexpr int KN = NP / 32;
  constexpr int ES = (int)sizeof(T);
  constexpr int VEC = 16 / ES;           // elements per 16-byte access
  constexpr int LDB = tr_ld(NP, ES);     // B tile: row reads and transposed reads
  constexpr int LDC = NP + VEC;          // C tile: row reads only
  constexpr int LDX = tr_ld(P, ES);      // X tile: transposed reads
  constexpr int LDM = kSub + 4;          // masked scores M[i][j]
  constexpr int LDH = NP + VEC;          // state copy for the state-term operand
  constexpr int NTI = kSub / 16;         // token tiles per sub-block
  constexpr int BRW = NP / VEC;          // 16-byte pieces per B/C row
  constexpr int XRW = P / VEC;           // 16-byte pieces per X row
  constexpr int BPT = (kSub * BRW + NTH - 1) / NTH;
  constexpr int XPT = (kSub * XRW + NTH - 1) / NTH;
  constexpr int NMT = 12;                // masked-score tile slots
  constexpr int MPW = (NMT + NW - 1) / NW;
  constexpr int NIT = NTI / KH;          // output token tiles per wave
  static_assert(NTILE % KH == 0 && NTI == 4, "tile split");

  __shared__ __attribute__((aligned(16))) T sB[kSub * LDB];
  __shared__ __attribute__((aligned(16))) T sC[kOut ? kSub * LDC : VEC];
  __shared__ __attribute__((aligned(16))) T sX[kSub * LDX];
  __shared__ __attribute__((aligned(16))) T sM[kOut ? kSub * LDM : VEC];
  __shared__ __attribute__((aligned(16))) T sH[(kOut && KH == 2) ? P * LDH : VEC];
  __shared__ float sC2[kSub]; // cum * log2(e)
  __shared__ float sQ2[kSub]; // cum * log2(e) - log2(Delta)   (+inf where Delta = 0)
  __shared__ float sW[kSub];  // exp(cum_last - cum_j) * Delta_j

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

  if (MODE == kWalkChunkState && seg == nseg - 1) return; // no consumer

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int pt = w % NPT, hv = w / NPT;
  const int prow = 16 * pt + li; // the state row this lane feeds as an operand

  const float a2 = prm.A[h] * kLog2e;
  const float d_h = prm.D ? prm.D[h] : 0.f;
  const float bias = (MODE == kWalkFull && prm.dt_bias) ? prm.dt_bias[h] : 0.f;
  const int64_t state_idx = ((int64_t)(ib * H + h) * nseg + seg) * P * N;

  // State tiles of this wave: hs[k][r] = S[p = prow][n = 16 (hv NTH2 + k) + 4 lg + r].
  f32x4 hs[NTH2];
#pragma unroll
  for (int k = 0; k < NTH2; ++k) hs[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (prm.init != nullptr) {
    const float *src = prm.init + state_idx + (int64_t)prow * N;
#pragma unroll
    for (int k = 0; k < NTH2; ++k) {
      const int n0 = 16 * (hv * NTH2 + k);
      if (n0 < N) hs[k] = *reinterpret_cast<const f32x4 *>(src + n0 + 4 * lg);
    }
  }
  // Publish the operand copy of the state (read after the loop's first barrier).
  auto publish_state = [&]() {
    if constexpr (kOut && KH == 2) {
#pragma unroll
      for (int k = 0; k < NTH2; ++k)
        st4<T>(&sH[prow * LDH + 16 * (hv * NTH2 + k) + 4 * lg], hs[k][0], hs[k][1], hs[k][2], hs[k][3]);
    }
  };
  publish_state();

  // Per-thread 16-byte pieces of the staged tiles: row and column within
  // the sub-block are fixed for the whole walk; only the base moves.
  const int64_t rowB = (int64_t)G * N;  // elements between consecutive tokens of B/C
  const int64_t rowX = (int64_t)H * P;  // ... of x and y
  const T *__restrict__ Bbase = reinterpret_cast<const T *>(prm.B) + ((int64_t)ib * L * G + g) * N;
  const T *__restrict__ Cbase = reinterpret_cast<const T *>(prm.C) + ((int64_t)ib * L * G + g) * N;
  const T *__restrict__ Xbase = reinterpret_cast<const T *>(prm.x) + (int64_t)ib * L * rowX + (int64_t)h * P;
  T *__restrict__ Ybase = reinterpret_cast<T *>(prm.out) + (int64_t)ib * L * rowX + (int64_t)h * P;
  // gate input of the output (out = y * silu(z)), or null
  const T *__restrict__ Zbase = prm.z ? reinterpret_cast<const T *>(prm.z) + (int64_t)ib * L * rowX + (int64_t)h * P
                                      : nullptr;
  const float *__restrict__ dtbase = (MODE == kWalkFull) ? prm.dt + (int64_t)ib * L * H + h
                                                         : prm.dt + (int64_t)(ib * H + h) * L;
  const int64_t dtstride = (MODE == kWalkFull) ? H : 1;

  float4 rB[BPT], rC[kOut ? BPT : 1], rX[XPT];
  float rdt = 0.f;
  // Loop-invariant byte offsets of this thread's 16-byte pieces inside a
  // tile; column padding (N < NP) points past the range and reads zero.
  constexpr uint32_t kOOB = 0x7ffffff0u;
  uint32_t offB[BPT], offX[XPT];
#pragma unroll
  for (int q = 0; q < BPT; ++q) {
    const int idx = tid + q * NTH;
    const int n0 = (idx % BRW) * VEC;
    offB[q] = (NP == N || n0 < N) ? (uint32_t)(((int64_t)(idx / BRW) * rowB + n0) * ES) : kOOB;
  }
#pragma unroll
  for (int q = 0; q < XPT; ++q) {
    const int idx = tid + q * NTH;
    offX[q] = (uint32_t)(((int64_t)(idx / XRW) * rowX + (idx % XRW) * VEC) * ES);
  }
  const uint32_t offDt = (uint32_t)(l * dtstride * 4);
  const uint32_t offY = (uint32_t)(((int64_t)li * rowX + 16 * pt + 4 * lg) * ES);
  // Loads of one sub-block, in three groups so that their issue spreads over
  // the compute phases of the previous sub-block.  Rows past the end of the
  // segment read as zero (buffer range check).
  auto fetch_x = [&](int t0, int nv) {
    const auto rsX = make_rsrc(Xbase + (int64_t)t0 * rowX, (uint32_t)(((int64_t)(nv - 1) * rowX + P) * ES));
    const auto rsD = make_rsrc(dtbase + (int64_t)t0 * dtstride, (uint32_t)(((int64_t)(nv - 1) * dtstride + 1) * 4));
#pragma unroll
    for (int q = 0; q < XPT; ++q)
      if (tid + q * NTH < kSub * XRW) rX[q] = bload16(rsX, offX[q]);
    rdt = bload4(rsD, offDt);
  };
  auto fetch_b = [&](int t0, int nv) {
    const auto rsB = make_rsrc(Bbase + (int64_t)t0 * rowB, (uint32_t)(((int64_t)(nv - 1) * rowB + N) * ES));
#pragma unroll
    for (int q = 0; q < BPT; ++q)
      if (tid + q * NTH < kSub * BRW) rB[q] = bload16(rsB, offB[q]);
  };
  auto fetch_c = [&](int t0, int nv) {
    if constexpr (kOut) {
      const auto rsC = make_rsrc(Cbase + (int64_t)t0 * rowB, (uint32_t)(((int64_t)(nv - 1) * rowB + N) * ES));
#pragma unroll
      for (int q = 0; q < BPT; ++q)
        if (tid + q * NTH < kSub * BRW) rC[q] = bload16(rsC, offB[q]);
    }
  };

  float seg_log2 = 0.f; // log2 decay of the segment so far
  int t0 = t_begin;
  int nv = min(kSub, t_end - t0);
  if (t0 < t_end) {
    fetch_x(t0, nv);
    fetch_b(t0, nv);
    fetch_c(t0, nv);
  }
  while (t0 < t_end) {
    __syncthreads(); // the previous sub-block is done with LDS

    // ---- stage the registers into row-major LDS tiles ---------------------
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      const int idx = tid + q * NTH;
      if (idx < kSub * BRW) {
        const int j = idx / BRW, n0 = (idx % BRW) * VEC;
        *reinterpret_cast<float4 *>(&sB[j * LDB + n0]) = rB[q];
        if (kOut) *reinterpret_cast<float4 *>(&sC[j * LDC + n0]) = rC[q];
      }
    }
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int idx = tid + q * NTH;
      if (idx < kSub * XRW) {
        const int j = idx / XRW, p0 = (idx % XRW) * VEC;
        *reinterpret_cast<float4 *>(&sX[j * LDX + p0]) = rX[q];
      }
    }
    {
      // Delta and the inclusive cumsum of Delta*A over the sub-block (wave
      // scan, lane = token), kept in log2 units.  Every wave computes the
      // same values and stores them (no wave-dependent branch in the loop).
      // Padding tokens get Delta = 0: no decay, no contribution.
      float dl = (MODE == kWalkFull) ? softplus_f(rdt + bias) : rdt;
      dl = (l < nv) ? dl : 0.f;
      const float c2 = wave_incl_scan(dl * a2);
      const float clast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c2), 63));
      sC2[l] = c2;
      sQ2[l] = c2 - hw_log2(dl);
      sW[l] = hw_exp2(clast - c2) * dl;
    }
    __syncthreads();

    const int t_next = t0 + kSub;
    const int nv_next = min(kSub, t_end - t_next);
    const bool more = t_next < t_end;
    if (more) fetch_x(t_next, nv_next);

    f32x4 yacc[NIT];
    if constexpr (kOut) {
      // ---- masked scores M[i][j] = (C_i . B_j) exp(cum_i - cum_j) Delta_j --
      //      = S^T[j][i] exp2(c2_i - q2_j); the diagonal also carries D, so
      //      the intra-block product adds D x_i.
      // All slots of a wave are computed without branches (the all-zero
      // tiles too, then masked), so their MFMA chains interleave.
      f32x4 macc[MPW];
#pragma unroll
      for (int k = 0; k < MPW; ++k) {
        const int slot = min(w + k * NW, NMT - 1);
        const int it = mtile_it(slot), jt = mtile_jt(slot);
        macc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KN; ++ks)
          macc[k] = mma(ld8(&sB[(16 * jt + li) * LDB + 32 * ks + 8 * lg]),
                        ld8(&sC[(16 * it + li) * LDC + 32 * ks + 8 * lg]), macc[k]);
      }
#pragma unroll
      for (int k = 0; k < MPW; ++k) {
        const int slot = w + k * NW;
        if (NMT % NW == 0 || slot < NMT) {
          const int it = mtile_it(slot), jt = mtile_jt(slot);
          const int i = 16 * it + li;
          const float ci = sC2[i];
          const float4 q4 = *reinterpret_cast<const float4 *>(&sQ2[16 * jt + 4 * lg]);
          float m[4] = {macc[k][0] * hw_exp2(ci - q4.x), macc[k][1] * hw_exp2(ci - q4.y),
                        macc[k][2] * hw_exp2(ci - q4.z), macc[k][3] * hw_exp2(ci - q4.w)};
          // causal mask (row tile it vs column tile jt), D on the diagonal
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int dj = 16 * jt + 4 * lg + r, di = 16 * it + li;
            m[r] = (dj < di) ? m[r] : (dj == di ? m[r] + d_h : 0.f);
          }
          st4<T>(&sM[i * LDM + 16 * jt + 4 * lg], m[0], m[1], m[2], m[3]);
        }
      }
      if (more) fetch_b(t_next, nv_next);

      // ---- state term: Y^T[p][i] = exp(cum_i) sum_n S[p][n] C[i][n] --------
      // A operand: the state rows of this p-tile, K = n in the order
      // {32ks + 4g + r, 32ks + 16 + 4g + r} that the register tiles hold.
      typename FragOf<T>::type hf[KN];
#pragma unroll
      for (int ks = 0; ks < KN; ++ks) {
        if constexpr (KH == 1) {
          float v[8];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            v[r] = hs[2 * ks][r];
            v[4 + r] = hs[2 * ks + 1][r];
          }
          hf[ks] = pack8<T>(v);
        } else {
          hf[ks] = ld4x2(&sH[prow * LDH + 32 * ks + 4 * lg], &sH[prow * LDH + 32 * ks + 16 + 4 * lg]);
        }
      }
#pragma unroll
      for (int u = 0; u < NIT; ++u) {
        const int i = 16 * (NIT * hv + u) + li;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KN; ++ks)
          acc = mma(hf[ks], ld4x2(&sC[i * LDC + 32 * ks + 4 * lg], &sC[i * LDC + 32 * ks + 16 + 4 * lg]),
                    acc);
        yacc[u] = acc * hw_exp2(sC2[i]);
      }
      if (more) fetch_c(t_next, nv_next);
      __syncthreads(); // M complete; every wave has read the state copy
    } else {
      if (more) fetch_b(t_next, nv_next);
    }

    // X^T fragments (rows p = prow, K = tokens), shared by the intra-block
    // product and the state update.
    typename FragOf<T>::type xf[kSub / 32];
#pragma unroll
    for (int ks = 0; ks < kSub / 32; ++ks) xf[ks] = trfrag(sX, LDX, 32 * ks, 16 * pt, li, lg);

    if constexpr (kOut) {
      // ---- intra-block term: Y^T[p][i] += sum_{j<=i} X^T[p][j] M[i][j] -----
      //      then store y (rows past the segment end fall outside the range)
      const auto rsY = make_rsrc(Ybase + (int64_t)t0 * rowX, (uint32_t)(((int64_t)(nv - 1) * rowX + P) * ES));
      const auto rsZ = make_rsrc(Zbase ? Zbase + (int64_t)t0 * rowX : Ybase,
                                 Zbase ? (uint32_t)(((int64_t)(nv - 1) * rowX + P) * ES) : 0u);
#pragma unroll
      for (int u = 0; u < NIT; ++u) {
        const int it = NIT * hv + u;
        const int i = 16 * it + li;
        if (KH == 2 && hv == 0) {
          yacc[u] = mma(xf[0], ld4x2(&sM[i * LDM + 4 * lg], &sM[i * LDM + 16 + 4 * lg]), yacc[u]);
        } else {
#pragma unroll
          for (int ks = 0; ks < (KH == 1 ? (16 * (u + 1) + 31) / 32 : 2); ++ks)
            yacc[u] = mma(xf[ks], ld4x2(&sM[i * LDM + 32 * ks + 4 * lg], &sM[i * LDM + 32 * ks + 16 + 4 * lg]),
                          yacc[u]);
        }
        f32x4 yv = yacc[u];
        if (Zbase) {
          const float4 zz = bload4x<T>(rsZ, offY + (uint32_t)(16 * it * rowX * ES));
          yv[0] *= silu_f(zz.x);
          yv[1] *= silu_f(zz.y);
          yv[2] *= silu_f(zz.z);
          yv[3] *= silu_f(zz.w);
        }
        bstore4<T>(rsY, offY + (uint32_t)(16 * it * rowX * ES), yv[0], yv[1], yv[2], yv[3]);
      }
    }

    // ---- state update: S^T = decay S^T + B^T (w o X) ------------------------
    seg_log2 += sC2[kSub - 1];
    const float dec = hw_exp2(sC2[kSub - 1]);
#pragma unroll
    for (int k = 0; k < NTH2; ++k) hs[k] *= dec;
#pragma unroll
    for (int ks = 0; ks < kSub / 32; ++ks) {
      const float4 wa = *reinterpret_cast<const float4 *>(&sW[32 * ks + 4 * lg]);
      const float4 wb = *reinterpret_cast<const float4 *>(&sW[32 * ks + 16 + 4 * lg]);
      const float v[8] = {elem(xf[ks], 0) * wa.x, elem(xf[ks], 1) * wa.y, elem(xf[ks], 2) * wa.z,
                          elem(xf[ks], 3) * wa.w, elem(xf[ks], 4) * wb.x, elem(xf[ks], 5) * wb.y,
                          elem(xf[ks], 6) * wb.z, elem(xf[ks], 7) * wb.w};
      const auto bx = pack8<T>(v);
#pragma unroll
      for (int k = 0; k < NTH2; ++k)
        hs[k] = mma(trfrag(sB, LDB, 32 * ks, 16 * (hv * NTH2 + k), li, lg), bx, hs[k]);
    }
    publish_state();
    t0 = t_next;
    nv = nv_next;
  }

  if (prm.seg_decay && tid == 0) prm.seg_decay[(int64_t)(ib * H + h) * nseg + seg] = seg_log2;
  float *dst = prm.state_out ? prm.state_out + state_idx
             : (prm.final_state && seg == nseg - 1) ? prm.final_state + (int64_t)(ib * H + h) * P * N
                                                     : nullptr;
  if (dst) {
#pragma unroll
    for (int k = 0; k < NTH2; ++k) {
      const int n0 = 16 * (hv * NTH2 + k);
      if (n0 < N) *reinterpret_cast<f32x4 *>(dst + (int64_t)prow * N + n0 + 4 * lg) = hs[k];
    }
  }
}

// ---------------------------------------------------------------------------
// Step sizes Delta = softplus(dt + bias), transposed to head-major [b, H, L]
// (the selective step size of the Mamba reading notes, selective-mechanism
// section).  One workgroup per (batch, 64-token tile, 64-head tile) stages
// dt through LDS: reads coalesce along heads, writes along tokens.
__global__ void __launch_bounds__(256)
delta_kernel(const float *__restrict__ dt, const float *__restrict__ dt_bias,
             float *__restrict__ delta, int b, int L, int H) {
  __shared__ float tile[64 * 65];
  const int ntt = (L + 63) / 64, nhb = (H + 63) / 64;
  const int hb = blockIdx.x % nhb;
  const int tt = (blockIdx.x / nhb) % ntt;
  const int ib = blockIdx.x / (nhb * ntt);
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int h0 = hb * 64, nh = min(64, H - h0);
  const int t0 = tt * 64, nv = min(64, L - t0);
  for (int idx = tid; idx < 64 * 64; idx += 256) {
    const int j = idx >> 6, hh = idx & 63;
    tile[j * 65 + hh] = (j < nv && hh < nh) ? dt[((int64_t)ib * L + t0 + j) * H + h0 + hh] : 0.f;
  }
  __syncthreads();
  for (int hh = w; hh < nh; hh += 4) {
    const int h = h0 + hh;
    if (l < nv)
      delta[((int64_t)ib * H + h) * L + t0 + l] = softplus_f(tile[l * 65 + hh] + (dt_bias ? dt_bias[h] : 0.f));
  }
}

// ---------------------------------------------------------------------------
// Inter-chunk state passing, sequential over chunks and parallel over
// (batch, head, P*N/4): each thread carries four consecutive fp32 state
// entries.  Slot c of `states` holds chunk c's own (zero-entry) end state on
// input and the state entering chunk c on output.  The chunk decays
// exp2(seg_decay) are read by lane c of a wave and broadcast with wave
// shuffles.  Four chunks' states are loaded before they are folded in, so
// the loads overlap the dependent multiply-add chain.
__global__ void __launch_bounds__(256)
state_pass_kernel(float *__restrict__ states, const float *__restrict__ seg_decay,
                  const float *__restrict__ init, int b, int H, int PN, int nc) {
  const int per_bh = PN / 4;
  const int64_t id = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t bh = id / per_bh;
  const int e4 = (int)(id % per_bh);
  const bool live = bh < (int64_t)b * H;
  const int lane = threadIdx.x & 63;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (live && init) s = reinterpret_cast<const float4 *>(init + bh * PN)[e4];
  float4 *base = reinterpret_cast<float4 *>(states + (live ? bh : 0) * (int64_t)nc * PN) + e4;
  const float *db = seg_decay + (live ? bh : 0) * (int64_t)nc;
  for (int c0 = 0; c0 < nc; c0 += 64) {
    // lane k holds the decay of chunk c0 + k
    const float my_dec = (c0 + lane < nc) ? hw_exp2(db[c0 + lane]) : 1.f;
    const int cnt = min(64, nc - c0);
    int k = 0;
    for (; k + 4 <= cnt; k += 4) {
      float4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        v[u] = (live && c0 + k + u + 1 < nc) ? base[(int64_t)(c0 + k + u) * per_bh] : make_float4(0, 0, 0, 0);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float d = __shfl(my_dec, k + u, 64);
        if (live) base[(int64_t)(c0 + k + u) * per_bh] = s;
        s.x = d * s.x + v[u].x; s.y = d * s.y + v[u].y;
        s.z = d * s.z + v[u].z; s.w = d * s.w + v[u].w;
      }
    }
    for (; k < cnt; ++k) {
      const float4 v = (live && c0 + k + 1 < nc) ? base[(int64_t)(c0 + k) * per_bh] : make_float4(0, 0, 0, 0);
      const float d = __shfl(my_dec, k, 64);
      if (live) base[(int64_t)(c0 + k) * per_bh] = s;
      s.x = d * s.x + v.x; s.y = d * s.y + v.y;
      s.z = d * s.z + v.z; s.w = d * s.w + v.w;
    }
  }
}

// ---------------------------------------------------------------------------
// Recurrent step ("From Transformer to Mamba", section 2.1, single-step
// update): one workgroup per (batch, head); N/4 threads per state row, each
// owning four consecutive entries; the readout sum over n is a DPP sum
// inside each 16-lane row, then shuffles across rows (N >= 128).  State and
// x go through range-checked buffer accesses (rows past P read zeros, their
// stores are dropped), so a batch of rows is loaded without branches and all
// its loads are in flight together; the state, read once and written once,
// streams non-temporally.
template <typename T> __device__ __forceinline__ float bload_elem(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ float bload_elem<__bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (float)__builtin_bit_cast(__bf16, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0));
}
template <> __device__ __forceinline__ float bload_elem<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return bload4(r, off);
}
template <typename T> __device__ __forceinline__ void bstore_elem(__amdgpu_buffer_rsrc_t r, uint32_t off, float v);
template <> __device__ __forceinline__ void bstore_elem<__bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, (__bf16)v), r, (int)off, 0, 0);
}
template <> __device__ __forceinline__ void bstore_elem<float>(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, (int)off, 0, 0);
}

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
  const auto rsS = make_rsrc(state + (int64_t)bh * P * N, (uint32_t)P * N * 4u);
  const auto rsX = make_rsrc(x + (int64_t)bh * P, (uint32_t)P * (uint32_t)sizeof(T));
  const auto rsO = make_rsrc(out + (int64_t)bh * P, (uint32_t)P * (uint32_t)sizeof(T));
  for (int p0 = 0; p0 < P; p0 += RPP * BATCH) {
    float4 s[BATCH];
    float xv[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int p = p0 + u * RPP + rp;
      s[u] = bload16_nt(rsS, (uint32_t)(p * TPR + c4) * 16u);
      xv[u] = bload_elem<T>(rsX, (uint32_t)p * (uint32_t)sizeof(T));
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
      if constexpr (TPR <= 16) {
        acc = lane_group_sum<TPR>(acc);
      } else {
        acc = lane_group_sum<16>(acc);
#pragma unroll
        for (int off = 16; off < TPR; off <<= 1) acc += __shfl_xor(acc, off, 64);
      }
      bstore16_nt(rsS, (uint32_t)(p * TPR + c4) * 16u, s[u]);
      // one lane per row writes y; the others aim past the range
      bstore_elem<T>(rsO, c4 == 0 ? (uint32_t)p * (uint32_t)sizeof(T) : 0xfffffff0u, acc + d_h * xv[u]);
    }
  }
}

template <typename T, int P, int N>
hipError_t launch_walk_t(WalkMode mode, const WalkParams &p, hipStream_t st) {
  const dim3 grid((unsigned)(p.b * p.H * p.nseg)), block(walk_waves<T, P>() * 64);
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
  case 128:
    // fp32 tiles for P = 128 exceed the 160 KB of LDS per workgroup.
    if constexpr (sizeof(T) == 2) return launch_walk_n<T, 128>(N, mode, p, st);
    return hipErrorInvalidValue;
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

hipError_t launch_delta(const float *dt, const float *dt_bias, float *delta, int b, int L, int H,
                        hipStream_t stream) {
  const int64_t n = (int64_t)b * ((L + 63) / 64) * ((H + 63) / 64);
  hipLaunchKernelGGL(delta_kernel, dim3((unsigned)n), dim3(256), 0, stream, dt, dt_bias, delta, b, L, H);
  return hipGetLastError();
}

hipError_t launch_state_pass(float *states, const float *seg_decay, const float *init, int b, int H,
                             int PN, int nc, hipStream_t stream) {
  const int64_t n = (int64_t)b * H * (PN / 4);
  hipLaunchKernelGGL(state_pass_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     states, seg_decay, init, b, H, PN, nc);
  return hipGetLastError();
}

hipError_t launch_step(int dtype, int N, float *state, const void *x, const float *dt,
                       const float *A, const void *B, const void *C, const float *D, void *out,
                       int b, int H, int P, int G, hipStream_t stream) {
  return dtype == 1 ? launch_step_t<__bf16>(N, state, x, dt, A, B, C, D, out, b, H, P, G, stream)
                    : launch_step_t<float>(N, state, x, dt, A, B, C, D, out, b, H, P, G, stream);
}

} // namespace ssd
