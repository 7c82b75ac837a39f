// ssd_quad.hip -- the whole-sequence quadratic form for short sequences
// (L <= 256): one launch, no state carried between blocks.
//
// The method ("Mamba-3 deep dive ch. 2, SSM foundations", 171host.com,
// section 2.2.1: the scan is one matrix product Y = (L o C B^T) X, whose mask
// entry L_ij is the product of the forget gates after j up to i; section
// 2.1.2 for the recurrence it equals; "Transformers are SSMs" summary,
// gongshangzheng.github.io, section 1.2: for a short sequence the quadratic,
// attention-like form is the cheap one).  With cum_i the inclusive sum of
// Delta*A up to token i (log2 units below) and an initial state S0:
//
//   y_i = sum_{j<=i} (C_i . B_j) 2^{cum_i - cum_j} Delta_j x_j + D x_i
//       + 2^{cum_i} S0 C_i
//   S_L = 2^{cum_last} S0 + sum_j 2^{cum_last - cum_j} Delta_j x_j B_j^T
//
// The exponents are taken per element (cum_i - cum_j <= 0 for j <= i), so no
// factor ever overflows and no renormalisation is needed.  cum is summed in
// fp64 and kept as an fp32 pair (hi, lo); an exponent is formed as
// (hi_i - hi_j) + (lo_i - lo_j) + log2 Delta_j, so it stays exact to fp32
// precision however far the decay runs (a single fp32 cum loses the
// difference of two large, nearly equal sums).
//
// Work split: one workgroup per (batch, head, 64-token query block iq).  Its
// NG groups of P/16 waves share the key blocks jb = 0..iq round-robin (group
// g takes jb = g, g + NG, ...); inside a group wave pt owns the output
// columns p in [16pt, 16pt+16).  Per key block a group stages B and X of the
// block in its own LDS area, builds the masked, decayed score tile
// M[i][j] = (C_i . B_j) 2^{cum_i - cum_j} Delta_j (with D on the diagonal)
// from matrix-core products, and accumulates Y^T += X^T M^T.  The query block
// of the last workgroup of a (batch, head) covers every key block, so that
// workgroup also forms the final state.  Group partials are summed in LDS in
// group order (deterministic).  All workgroups run at once: the critical path
// is one query block (NG-fold parallel over its key blocks), not the chain of
// blocks a walk follows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kQuadLds = 160 * 1024;

// Inclusive prefix sum of an fp64 value over the 64 lanes of a wave: the
// row shifts and row broadcasts of wave_incl_scan applied to both 32-bit
// halves.
__device__ __forceinline__ double wave_incl_scan_f64(double v) {
#define SSD_DPP64(ctrl, rmask, bound)                                                              \
  {                                                                                                \
    const uint64_t u = __builtin_bit_cast(uint64_t, v);                                            \
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, ctrl, rmask, 0xf, bound);      \
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), ctrl, rmask, 0xf, bound); \
    v += __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);               \
  }
  SSD_DPP64(0x111, 0xf, true)
  SSD_DPP64(0x112, 0xf, true)
  SSD_DPP64(0x114, 0xf, true)
  SSD_DPP64(0x118, 0xf, true)
  SSD_DPP64(0x142, 0xa, false)
  SSD_DPP64(0x143, 0xc, false)
#undef SSD_DPP64
  return v;
}

template <typename T, int P, int N> struct QuadShape {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int VEC = 16 / ES;          // elements per 16-byte piece
  static constexpr int NP = (N + 31) / 32 * 32; // N padded to a K-step
  static constexpr int NTILE = NP / 16;
  static constexpr int KN = NP / 32;
  static constexpr int NPT = P / 16;           // waves per group (p-tiles)
  static constexpr int LDB = tr_ld(NP, ES);    // B: row and transposed reads
  static constexpr int LDC = NP + VEC;         // C: row reads
  static constexpr int LDX = tr_ld(P, ES);     // X: transposed reads
  static constexpr int LDM = 64 + 4;           // masked scores M[i][j]
  static constexpr int C_BYTES = 64 * LDC * ES;
  static constexpr int FIX_BYTES = 256 * 8 + 4 * 8 + 3 * 256 * 4; // cum (fp64), block sums, hi, lo, log2 Delta
  static constexpr int GB = ((64 * LDB + 64 * LDX + 64 * LDM) * ES + 15) / 16 * 16; // one group area
  static constexpr int RED_BYTES = 64 * P * 4 + P * NP * 4; // fp32 y and final-state sums
  static constexpr int fits(int ng) {
    return C_BYTES + FIX_BYTES + ng * GB <= kQuadLds && (ng == 1 || ng * GB >= RED_BYTES) &&
           ng * NPT <= 16; // at most 1024 threads
  }
  static constexpr int NG = fits(4) ? 4 : fits(2) ? 2 : 1;
  static constexpr int NW = NG * NPT;
  static constexpr int NTH = NW * 64;
  static constexpr int BYTES = C_BYTES + FIX_BYTES + NG * GB;
  static_assert(fits(NG), "quadratic path does not fit the LDS");
};

template <typename T, int P, int N>
__global__ void __launch_bounds__((QuadShape<T, P, N>::NTH)) quad_kernel(const WalkParams prm) {
  using S = QuadShape<T, P, N>;
  constexpr int ES = S::ES, VEC = S::VEC, NP = S::NP, NTILE = S::NTILE, KN = S::KN, NPT = S::NPT;
  constexpr int LDB = S::LDB, LDC = S::LDC, LDX = S::LDX, LDM = S::LDM, NG = S::NG, NTH = S::NTH;
  constexpr int TPW = 16 / NPT;     // score tiles per wave and key block
  constexpr int TCH = TPW < 4 ? TPW : 4; // score tiles computed together
  constexpr int BRW = NP / VEC, XRW = P / VEC;
  constexpr int GTH = NPT * 64;     // threads of a group
  constexpr uint32_t kOOB = 0x7ffffff0u;

  __shared__ __attribute__((aligned(16))) unsigned char smem[S::BYTES];
  T *sC = reinterpret_cast<T *>(smem);
  double *sCd = reinterpret_cast<double *>(smem + S::C_BYTES); // cum (log2, fp64), token-indexed
  double *sTot = sCd + 256;                                     // per-block sums of Delta*A (log2)
  float *sHi = reinterpret_cast<float *>(sTot + 4);             // cum = hi + lo
  float *sLo = sHi + 256;
  float *sLg = sLo + 256;                                       // log2 Delta (-inf at Delta = 0)
  unsigned char *gbase = smem + S::C_BYTES + S::FIX_BYTES;

  const int H = prm.H, G = prm.G, L = prm.L;
  const int nq = (L + 63) / 64;
  const int BH = prm.b * H;
  // heaviest query blocks (the last ones) first
  const int bid = blockIdx.x;
  const int iq = nq - 1 - bid / BH;
  const int ib = (bid % BH) / H, h = bid % H;
  const int g = (int)((int64_t)h * G / H);
  const int tid = threadIdx.x, l = tid & 63, li = l & 15, lg = l >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = w / NPT, pt = w % NPT;
  const int gtid = tid - grp * GTH;
  const bool last_q = iq == nq - 1;
  const bool want_final = last_q && prm.final_state != nullptr;
  const int q0 = 64 * iq;
  const int nvq = min(64, L - q0);

  T *sB = reinterpret_cast<T *>(gbase + grp * S::GB);
  T *sX = sB + 64 * LDB;
  T *sM = sX + 64 * LDX;

  const float a2 = prm.A[h] * kLog2e;
  const float d_h = prm.D ? prm.D[h] : 0.f;
  const float bias = prm.dt_bias ? prm.dt_bias[h] : 0.f;
  const int64_t rowB = (int64_t)G * N, rowX = (int64_t)H * P;
  const T *Bbase = reinterpret_cast<const T *>(prm.B) + ((int64_t)ib * L * G + g) * N;
  const T *Cbase = reinterpret_cast<const T *>(prm.C) + ((int64_t)ib * L * G + g) * N;
  const T *Xbase = reinterpret_cast<const T *>(prm.x) + (int64_t)ib * L * rowX + (int64_t)h * P;
  const float *dtbase = prm.dt + (int64_t)ib * L * H + h;

  // ---- every global load of the first round is issued up front -----------
  constexpr int CPT = (64 * BRW + NTH - 1) / NTH;  // C pieces per thread
  constexpr int BPT = (64 * BRW + GTH - 1) / GTH;  // B pieces per group thread
  constexpr int XPT = (64 * XRW + GTH - 1) / GTH;  // X pieces per group thread
  constexpr int DPW = (4 + S::NW - 1) / S::NW;     // step-size blocks per wave
  float rdt[DPW];
#pragma unroll
  for (int k = 0; k < DPW; ++k) {
    const int t = 64 * (w + k * S::NW) + l;
    rdt[k] = (w + k * S::NW <= iq && t < L) ? dtbase[(int64_t)t * H] : 0.f;
  }
  float4 rC[CPT], rB[BPT], rX[XPT];
  {
    const auto rsC = make_rsrc(Cbase + (int64_t)q0 * rowB, (uint32_t)(((int64_t)(nvq - 1) * rowB + N) * ES));
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int idx = tid + q * NTH, j = idx / BRW, n0 = (idx % BRW) * VEC;
      const uint32_t off = (idx < 64 * BRW && (NP == N || n0 < N)) ? (uint32_t)(((int64_t)j * rowB + n0) * ES) : kOOB;
      rC[q] = bload16(rsC, off);
    }
  }
  // B and X of key block jb into this thread's registers (rows past L and
  // pieces past the tile read zero)
  auto load_bx = [&](int jb) {
    const int t0 = 64 * jb, nv = min(64, L - t0);
    const auto rsB = make_rsrc(Bbase + (int64_t)t0 * rowB, (uint32_t)(((int64_t)(nv - 1) * rowB + N) * ES));
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      const int idx = gtid + q * GTH, j = idx / BRW, n0 = (idx % BRW) * VEC;
      const uint32_t off = (idx < 64 * BRW && (NP == N || n0 < N)) ? (uint32_t)(((int64_t)j * rowB + n0) * ES) : kOOB;
      rB[q] = bload16(rsB, off);
    }
    const auto rsX = make_rsrc(Xbase + (int64_t)t0 * rowX, (uint32_t)(((int64_t)(nv - 1) * rowX + P) * ES));
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int idx = gtid + q * GTH, j = idx / XRW, p0 = (idx % XRW) * VEC;
      rX[q] = bload16(rsX, idx < 64 * XRW ? (uint32_t)(((int64_t)j * rowX + p0) * ES) : kOOB);
    }
  };
  auto store_bx = [&]() {
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      const int idx = gtid + q * GTH;
      if (idx < 64 * BRW) *reinterpret_cast<float4 *>(&sB[(idx / BRW) * LDB + (idx % BRW) * VEC]) = rB[q];
    }
#pragma unroll
    for (int q = 0; q < XPT; ++q) {
      const int idx = gtid + q * GTH;
      if (idx < 64 * XRW) *reinterpret_cast<float4 *>(&sX[(idx / XRW) * LDX + (idx % XRW) * VEC]) = rX[q];
    }
  };
  if (grp <= iq) load_bx(grp);

  // ---- step sizes and cumulative log2 decay of tokens [0, 64 (iq + 1)) -----
#pragma unroll
  for (int k = 0; k < DPW; ++k) {
    const int jb = w + k * S::NW;
    if (jb <= iq) {
      const int t = 64 * jb + l;
      float dl = softplus_f(rdt[k] + bias);
      dl = t < L ? dl : 0.f; // padding tokens: no decay, no contribution
      const double c = wave_incl_scan_f64((double)(dl * a2));
      sCd[t] = c;
      sLg[t] = hw_log2(dl);
      if (l == 63) sTot[jb] = c;
    }
  }
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int idx = tid + q * NTH;
    if (idx < 64 * BRW) *reinterpret_cast<float4 *>(&sC[(idx / BRW) * LDC + (idx % BRW) * VEC]) = rC[q];
  }
  if (grp <= iq) store_bx();
  __syncthreads();
  for (int t = tid; t < 64 * (iq + 1); t += NTH) {
    double c = sCd[t];
    for (int k = 0; k < t / 64; ++k) c += sTot[k];
    const float hi = (float)c;
    sHi[t] = hi;
    sLo[t] = (float)(c - (double)hi);
  }
  __syncthreads();
  // log2 weight of key j for query i (j <= i): cum_i - cum_j + log2 Delta_j
  auto expo = [&](float hi_i, float lo_i, int j) { return (hi_i - sHi[j]) + (lo_i - sLo[j]) + sLg[j]; };
  const int tl = L - 1 < 64 * (iq + 1) ? L - 1 : 0;
  const float hi_last = sHi[tl], lo_last = sLo[tl];

  // ---- key blocks, NG at a time --------------------------------------------
  f32x4 yacc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) yacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 hs[NTILE]; // final state rows [16pt, 16pt+16) (last query block only)
#pragma unroll
  for (int k = 0; k < NTILE; ++k) hs[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int rounds = (iq + NG) / NG;
  for (int r = 0; r < rounds; ++r) {
    const int jb = grp + r * NG;
    const bool act = jb <= iq;
    if (r > 0) {
      if (act) store_bx();
      __syncthreads();
    }
    // the next round's key block loads overlap this round's products
    if (jb + NG <= iq) load_bx(jb + NG);
    if (act) {
      // masked, decayed score tiles (it, jt): M[i][j] for query rows
      // 16it + li and key columns 16jt + 4lg + r; wave pt builds tiles
      // [TPW pt, TPW (pt + 1)).
      const bool diag = jb == iq;
#pragma unroll
      for (int tc = 0; tc < TPW; tc += TCH) {
        f32x4 macc[TCH];
#pragma unroll
        for (int k = 0; k < TCH; ++k) {
          const int s = TPW * pt + tc + k, it = s / 4, jt = s % 4;
          macc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (!(diag && jt > it)) {
#pragma unroll
            for (int ks = 0; ks < KN; ++ks)
              macc[k] = mma(ld8(&sB[(16 * jt + li) * LDB + 32 * ks + 8 * lg]),
                            ld8(&sC[(16 * it + li) * LDC + 32 * ks + 8 * lg]), macc[k]);
          }
        }
#pragma unroll
        for (int k = 0; k < TCH; ++k) {
          const int s = TPW * pt + tc + k, it = s / 4, jt = s % 4;
          const int i = 16 * it + li;
          const float hi_i = sHi[q0 + i], lo_i = sLo[q0 + i];
          float m[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int j = 16 * jt + 4 * lg + rr;
            const float v = macc[k][rr] * hw_exp2(expo(hi_i, lo_i, 64 * jb + j));
            m[rr] = (!diag || j < i) ? v : (j == i ? v + d_h : 0.f);
          }
          st4<T>(&sM[i * LDM + 16 * jt + 4 * lg], m[0], m[1], m[2], m[3]);
        }
      }
    }
    __syncthreads();
    if (act) {
      typename FragOf<T>::type xf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) xf[ks] = trfrag(sX, LDX, 32 * ks, 16 * pt, li, lg);
      // Y^T[p][i] += sum_j X^T[p][j] M[i][j]
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 16 * u + li;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          yacc[u] = mma(xf[ks], ld4x2(&sM[i * LDM + 32 * ks + 4 * lg], &sM[i * LDM + 32 * ks + 16 + 4 * lg]), yacc[u]);
      }
      if (want_final) {
        // S^T += B^T (w o X), w_j = 2^{cum_last - cum_j} Delta_j
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int jbase = 64 * jb + 32 * ks + 4 * lg;
          float v[8];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            v[rr] = elem(xf[ks], rr) * hw_exp2(expo(hi_last, lo_last, jbase + rr));
            v[4 + rr] = elem(xf[ks], 4 + rr) * hw_exp2(expo(hi_last, lo_last, jbase + 16 + rr));
          }
          const auto bx = pack8<T>(v);
#pragma unroll
          for (int k = 0; k < NTILE; ++k) hs[k] = mma(trfrag(sB, LDB, 32 * ks, 16 * k, li, lg), bx, hs[k]);
        }
      }
    }
    __syncthreads(); // the group area is rewritten next round
  }

  // ---- initial-state terms (group 0) ---------------------------------------
  if (prm.init != nullptr && grp == 0) {
    const float *src = prm.init + ((int64_t)(ib * H + h) * P + 16 * pt + li) * N;
    f32x4 s0[NTILE];
#pragma unroll
    for (int k = 0; k < NTILE; ++k)
      s0[k] = (16 * k < N) ? *reinterpret_cast<const f32x4 *>(src + 16 * k + 4 * lg) : f32x4{0.f, 0.f, 0.f, 0.f};
    // y_i += 2^{cum_i} S0 C_i: A operand = rows of S0, K = n
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = 16 * u + li;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KN; ++ks) {
        float v[8];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          v[rr] = s0[2 * ks][rr];
          v[4 + rr] = s0[2 * ks + 1][rr];
        }
        acc = mma(pack8<T>(v), ld4x2(&sC[i * LDC + 32 * ks + 4 * lg], &sC[i * LDC + 32 * ks + 16 + 4 * lg]), acc);
      }
      yacc[u] += acc * hw_exp2(sHi[q0 + i] + sLo[q0 + i]);
    }
    if (want_final) {
      const float dec = hw_exp2(hi_last + lo_last);
#pragma unroll
      for (int k = 0; k < NTILE; ++k) hs[k] += s0[k] * dec;
    }
  }

  // ---- sums over the groups (in group order), then the stores --------------
  T *Ybase = reinterpret_cast<T *>(prm.out) + ((int64_t)ib * L + q0) * rowX + (int64_t)h * P;
  const T *Zbase = prm.z ? reinterpret_cast<const T *>(prm.z) + ((int64_t)ib * L + q0) * rowX + (int64_t)h * P
                         : nullptr;
  float *fin = want_final ? prm.final_state + (int64_t)(ib * H + h) * P * N : nullptr;
  if constexpr (NG == 1) {
    const auto rsY = make_rsrc(Ybase, (uint32_t)(((int64_t)(nvq - 1) * rowX + P) * ES));
    const auto rsZ = make_rsrc(Zbase ? Zbase : Ybase, Zbase ? (uint32_t)(((int64_t)(nvq - 1) * rowX + P) * ES) : 0u);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t off = (uint32_t)(((int64_t)(16 * u + li) * rowX + 16 * pt + 4 * lg) * ES);
      f32x4 yv = yacc[u];
      if (Zbase) {
        const float4 zz = bload4x<T>(rsZ, off);
        yv[0] *= silu_f(zz.x);
        yv[1] *= silu_f(zz.y);
        yv[2] *= silu_f(zz.z);
        yv[3] *= silu_f(zz.w);
      }
      bstore4<T>(rsY, off, yv[0], yv[1], yv[2], yv[3]);
    }
    if (fin) {
#pragma unroll
      for (int k = 0; k < NTILE; ++k)
        if (16 * k < N) *reinterpret_cast<f32x4 *>(fin + (int64_t)(16 * pt + li) * N + 16 * k + 4 * lg) = hs[k];
    }
  } else {
    float *sYr = reinterpret_cast<float *>(gbase);  // [64 tokens][P]
    float *sFr = sYr + 64 * P;                       // [P][NP]
    for (int k = 0; k < NG; ++k) {
      if (grp == k) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int i = 16 * u + li;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            float *d = &sYr[i * P + 16 * pt + 4 * lg + rr];
            *d = (k == 0 ? 0.f : *d) + yacc[u][rr];
          }
        }
        if (want_final) {
#pragma unroll
          for (int kk = 0; kk < NTILE; ++kk) {
            float *d = &sFr[(16 * pt + li) * NP + 16 * kk + 4 * lg];
            f32x4 v = hs[kk];
            if (k != 0) v += *reinterpret_cast<f32x4 *>(d);
            *reinterpret_cast<f32x4 *>(d) = v;
          }
        }
      }
      __syncthreads();
    }
    const auto rsY = make_rsrc(Ybase, (uint32_t)(((int64_t)(nvq - 1) * rowX + P) * ES));
    const auto rsZ = make_rsrc(Zbase ? Zbase : Ybase, Zbase ? (uint32_t)(((int64_t)(nvq - 1) * rowX + P) * ES) : 0u);
    for (int idx = tid; idx < 64 * (P / 4); idx += NTH) {
      const int i = idx / (P / 4), p0 = 4 * (idx % (P / 4));
      const float4 v4 = *reinterpret_cast<const float4 *>(&sYr[i * P + p0]);
      float v[4] = {v4.x, v4.y, v4.z, v4.w};
      const uint32_t off = (uint32_t)(((int64_t)i * rowX + p0) * ES);
      if (Zbase) {
        const float4 zz = bload4x<T>(rsZ, off);
        v[0] *= silu_f(zz.x);
        v[1] *= silu_f(zz.y);
        v[2] *= silu_f(zz.z);
        v[3] *= silu_f(zz.w);
      }
      bstore4<T>(rsY, off, v[0], v[1], v[2], v[3]);
    }
    if (fin) {
      for (int idx = tid; idx < P * (N / 4); idx += NTH) {
        const int p = idx / (N / 4), n0 = 4 * (idx % (N / 4));
        *reinterpret_cast<float4 *>(fin + (int64_t)p * N + n0) = *reinterpret_cast<const float4 *>(&sFr[p * NP + n0]);
      }
    }
  }
}

template <typename T, int P>
hipError_t launch_quad_p(int N, const WalkParams &p, hipStream_t st) {
  const int nq = (p.L + 63) / 64;
  const dim3 grid((unsigned)(p.b * p.H * nq));
  switch (N) {
#define SSD_QUAD_N(NN)                                                                              \
  case NN:                                                                                          \
    hipLaunchKernelGGL((quad_kernel<T, P, NN>), grid, dim3(QuadShape<T, P, NN>::NTH), 0, st, p);    \
    return hipGetLastError();
    SSD_QUAD_N(16)
    SSD_QUAD_N(32)
    SSD_QUAD_N(64)
    SSD_QUAD_N(128)
#undef SSD_QUAD_N
  default: return hipErrorInvalidValue;
  }
}

} // namespace

hipError_t launch_quad(int dtype, int P, int N, const WalkParams &p, hipStream_t stream) {
  if (p.L < 1 || p.L > kQuadMaxL) return hipErrorInvalidValue;
  if (dtype == 1) {
    switch (P) {
    case 16: return launch_quad_p<__bf16, 16>(N, p, stream);
    case 32: return launch_quad_p<__bf16, 32>(N, p, stream);
    case 64: return launch_quad_p<__bf16, 64>(N, p, stream);
    case 128: return launch_quad_p<__bf16, 128>(N, p, stream);
    default: return hipErrorInvalidValue;
    }
  }
  switch (P) {
  case 16: return launch_quad_p<float, 16>(N, p, stream);
  case 32: return launch_quad_p<float, 32>(N, p, stream);
  case 64: return launch_quad_p<float, 64>(N, p, stream);
  default: return hipErrorInvalidValue;
  }
}

} // namespace ssd
