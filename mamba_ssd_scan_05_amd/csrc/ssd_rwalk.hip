// ssd_rwalk.hip -- the row-sliced walk for bf16 inputs.
//
// The method ("Mamba-3 deep dive ch. 2, SSM foundations", 171host.com,
// section 2.1.2 recurrence, section 2.2.1 matrix form Y = (L o C B^T) X;
// "Transformers are SSMs" summary, gongshangzheng.github.io, sections
// 1.1-1.2: blocks evaluated with the quadratic form, linked through the
// N-dimensional state).  For a 64-token sub-block after state S (P x N),
// c_t = log2-scaled inclusive cumsum of Delta*A, q_t = c_t - log2(Delta_t):
//
//   y_t = 2^{c_t} S C_t + sum_{t'<=t} 2^{c_t - q_t'} (C_t . B_t') x_t' + D x_t
//   S'  = 2^{c_last} S + sum_t 2^{c_last - q_t} x_t B_t^T
//
// Two observations shape this kernel:
//
// 1. The raw scores C_t . B_t' do not depend on the head, only on its B/C
//    group.  prep_kernel (ssd_prep.hip) computes them once per (batch,
//    group, sub-block) as a causal 64x64 bf16 tile, next to the C and B
//    tiles, all in matrix-core fragment order (the sub-block's record);
//    every head of the group reads that record.
//
// 2. The decay weight is separable: 2^{c_t - q_t'} = 2^{c_t + e} 2^{-q_t' - e}
//    for any reference e.  The kernel keeps the state as S = 2^e hs, where
//    hs is the register tile and e a running wave-uniform exponent; then
//       y_t = 2^{c_t + e} [ hs C_t + sum_t' Score[t][t'] xs_t' ] + D x_t,
//       xs_t' = 2^{-q_t' - e} x_t',   hs' = hs + sum_t xs_t B_t^T,
//       e' = e + c_last,
//    so the intra-block product takes the shared score tile as it is, the
//    decay becomes a per-token scale of x and of y, and the register tile is
//    never rescaled except when e drifts out of range (an exact shift by
//    whole octaves).  Both token factors stay within 2^{+-kExpLim} while the
//    sub-block's decay span |c_last| is at most kSpanMax; longer spans take
//    the per-element form (slow path).
//
// Work split: a workgroup of W waves owns 16W consecutive state rows of one
// (batch, group) -- rows are (head, p) pairs of the heads in the group, 16
// rows per wave, all in one head -- and walks the sequence in 64-token
// sub-blocks.  The B and C fragments of a sub-block's record are copied
// once into LDS and read by every wave (one 16-byte read per fragment);
// each wave holds its 16 x N state in MFMA accumulator registers, stages
// its own 16 columns of x in a private LDS tile and loads the score
// fragments of the record straight from global memory (L2).  Two schedules of
// the same arithmetic (bitwise the same results): with at most four waves
// every wave has a SIMD to itself and the plain order is fastest; with more,
// the decay factors of the next sub-block are computed next to the products
// of the current one.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

// Decay span |c_last| (log2 units) up to which a sub-block takes the
// separable form, and the bound on the state exponent e: with e kept in
// [|c_last| - kExpLim, kExpLim] every token factor 2^{c + e} and
// 2^{log2 Delta - c - e} lies within 2^{+-kExpLim} (times Delta), far inside
// the fp32 / bf16 exponent range, and so do the products they enter.
constexpr float kSpanMax = 178.f;
constexpr float kExpLim = 90.f;

// Position of K-value j (0..7) of lane group g inside a 32-column group, in
// the order the transposed fragments use: {4g .. 4g+3, 16+4g .. 16+4g+3}.
// The score tile is stored with its columns permuted so that these eight
// values are contiguous: column 32ks + 8g + j holds t' = 32ks + kperm(g, j).
__host__ __device__ constexpr int kperm(int g, int j) { return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4); }

// ---------------------------------------------------------------------------
// The row-sliced walk.
// This file is built with MFMA accumulators in ordinary VGPRs: with
// accumulator registers the compiler parks the state tile there and copies
// it to VGPRs and back every sub-block.
// GATED: out = y * silu(z) with z read next to y.
template <int N, int W, bool GATED>
__global__ void __launch_bounds__(W * 64) rwalk_kernel(const RWalkParams prm) {
  constexpr int NTH = W * 64;
  constexpr int NT = N / 16;            // n-tiles of the state
  constexpr int KN = N / 32;            // K-steps over n
  constexpr int NCB = 4 * KN;           // C fragment blocks of a record
  constexpr int NBB = 2 * NT;           // B fragment blocks of a record
  constexpr int NRB = NCB + NBB + 6;    // blocks per record (C, B, scores)
  constexpr int PIECES = (NCB + NBB) * 64; // 16-byte pieces staged per sub-block
  constexpr int PPT = (PIECES + NTH - 1) / NTH;
  constexpr int NSF = 6;                // score fragments per lane and sub-block

  // C and B fragment blocks of a sub-block's record, double-buffered: a
  // fragment is the 16 bytes of its lane, one conflict-free LDS read
  __shared__ __attribute__((aligned(16))) __bf16 sRec[2][(NCB + NBB) * 512];
  __shared__ __attribute__((aligned(16))) __bf16 sX[W][64 * 16]; // x[token][16 columns]
  // per-wave token factors, double-buffered: scan() fills the other slot
  __shared__ __attribute__((aligned(16))) float sF0[2][W][64];   // xs scale (fast) / w (slow)
  __shared__ __attribute__((aligned(16))) float sF1[2][W][64];   // y scale 2^{c + e}
  __shared__ __attribute__((aligned(16))) float2 sQC[2][W][64];  // (q, c) for the slow path
  // With more than four waves: y of a sub-block for all rows of the
  // workgroup, [token][row], written by each wave and stored after the next
  // barrier as whole row runs.
  constexpr int YLD = 16 * W + 8;
  __shared__ __attribute__((aligned(16))) __bf16 sY[2][(W > 4 ? 64 : 1) * YLD];

  const int H = prm.H, G = prm.G, L = prm.L, P = prm.P;
  const int nwg = gridDim.x, bid = blockIdx.x;
  // XCD-aware order: consecutive ids go round-robin to the 8 XCDs; give
  // each XCD a contiguous range of logical ids so that the workgroups of one
  // (batch, group) share its B/C/score tiles through one L2.
  const int logical = (nwg % 8 == 0) ? (bid % 8) * (nwg / 8) + bid / 8 : bid;
  const int bg = logical / prm.wg_per_bg, wi = logical % prm.wg_per_bg;
  const int g = bg % G, ib = bg / G;
  const int tid = threadIdx.x, l = tid & 63, li = l & 15, lg = l >> 4;
  // The wave index is uniform across the wave; readfirstlane makes that
  // visible to the compiler, so that every per-wave address, buffer
  // descriptor and branch below lives in scalar registers.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int R = (wi * W + w) * 16;
  const bool active = R < prm.rows_per_bg;
  const int Rc = active ? R : 0;
  const int h = g * (H / G) + Rc / P;
  const int p0 = Rc % P;

  const float a2 = prm.A[h] * kLog2e;
  const float d_h = prm.D ? prm.D[h] : 0.f;
  const float bias = prm.dt_bias ? prm.dt_bias[h] : 0.f;
  const int64_t srow = ((int64_t)(ib * H + h) * P + p0 + li) * N; // state row p0 + li

  // hs[k][r] = S[p0 + li][16k + 4lg + r]
  f32x4 hs[NT];
#pragma unroll
  for (int k = 0; k < NT; ++k) hs[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (prm.init != nullptr && active) {
#pragma unroll
    for (int k = 0; k < NT; ++k) hs[k] = *reinterpret_cast<const f32x4 *>(prm.init + srow + 16 * k + 4 * lg);
  }

  const int64_t rowX = (int64_t)H * P;
  const __bf16 *Xbase = reinterpret_cast<const __bf16 *>(prm.x) + (int64_t)ib * L * rowX + (int64_t)h * P + p0;
  const float *dtbase = prm.dt + (int64_t)ib * L * H + h;
  const int nsub = (L + 63) / 64;
  // records of this (batch, group), one per sub-block
  const __bf16 *Rbase = reinterpret_cast<const __bf16 *>(prm.rec) + (int64_t)bg * nsub * (NRB * 512);

  // Loop-invariant offsets.  Every wave issues the same sequence of memory
  // operations on every path through the loop (threads without a piece of
  // their own repeat the last piece; fetches past the end use empty ranges
  // and read zeros; stores of idle waves fall outside an empty range), so
  // the compiler can wait for exactly the loads each step needs while
  // later loads and the y stores stay in flight.
  uint32_t offR[PPT];
#pragma unroll
  for (int i = 0; i < PPT; ++i) offR[i] = (uint32_t)min(tid + i * NTH, PIECES - 1) * 16u;
  // x pieces of this wave: piece l + 64e = (token, half) -> 8 columns.
  uint32_t offX[2];
  int ldsX[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int pc = l + 64 * e, tok = pc >> 1, half = pc & 1;
    offX[e] = (uint32_t)((tok * rowX + 8 * half) * 2);
    ldsX[e] = tok * 16 + 8 * half;
  }
  float4 rR[PPT], rX[2];
  // B, C and x of sub-block k (loads past the end read zeros).  With more
  // than four waves the byte counts are formed before the select, which
  // makes the choice a scalar select and keeps the loop body one scheduling
  // region; with one wave per SIMD the branch form schedules better (both
  // measured; the gated walk keeps the branch form as well).
  auto fetch_bcx = [&](int k) {
    const int t0 = 64 * k, nv = min(64, L - t0);
    const uint32_t bcb = nv > 0 ? (uint32_t)PIECES * 16u : 0u;
    const auto rsR = make_rsrc(Rbase + (int64_t)min(k, nsub - 1) * (NRB * 512), bcb);
#pragma unroll
    for (int i = 0; i < PPT; ++i) rR[i] = bload16(rsR, offR[i]);
    uint32_t nbX;
    if constexpr (W > 4 && !GATED) {
      const uint32_t nbX0 = (uint32_t)(((int64_t)(nv - 1) * rowX + 16) * 2);
      nbX = nv > 0 ? nbX0 : 0u;
    } else {
      nbX = nv > 0 ? (uint32_t)(((int64_t)(nv - 1) * rowX + 16) * 2) : 0u;
    }
    const auto rsX = make_rsrc(Xbase + (int64_t)t0 * rowX, nbX);
    rX[0] = bload16(rsX, offX[0]);
    rX[1] = bload16(rsX, offX[1]);
  };
  // Raw step size of token l of sub-block k (zero past the end).
  auto fetch_dt = [&](int k) {
    const int t0 = 64 * k, nv = min(64, L - t0);
    const auto rsD = make_rsrc(dtbase + (int64_t)t0 * H, nv > 0 ? (uint32_t)(((int64_t)(nv - 1) * H + 1) * 4) : 0u);
    return bload4(rsD, (uint32_t)(l * H * 4));
  };
  // Score fragments of sub-block k, issued right after the previous
  // sub-block's intra-block product has consumed the registers.
  FragBF sf[NSF];
  auto fetch_scores = [&](int k) {
    const auto rsS = make_rsrc(Rbase + (int64_t)k * (NRB * 512) + (NCB + NBB) * 512, NSF * 1024u);
#pragma unroll
    for (int f = 0; f < NSF; ++f) sf[f].v = __builtin_bit_cast(bf16x8, bload16(rsS, (uint32_t)(f * 1024 + 16 * l)));
  };
  auto stage = [&](int slot) {
#pragma unroll
    for (int i = 0; i < PPT; ++i) *reinterpret_cast<float4 *>(&sRec[slot][offR[i] / 2]) = rR[i];
    *reinterpret_cast<float4 *>(&sX[w][ldsX[0]]) = rX[0];
    *reinterpret_cast<float4 *>(&sX[w][ldsX[1]]) = rX[1];
  };

  // ---- decay factors of one sub-block (lane = token) ------------------------
  // The state is kept as S = 2^e * hs with a wave-uniform exponent e, so that
  // the separable path never rescales the register tile: with e_k the
  // exponent in force during sub-block k,
  //   y_t = 2^{c_t + e_k} [ hs C_t + sum_t' Score[t][t'] xs_t' ] + D x_t,
  //   xs_t = 2^{-q_t - e_k} x_t,   hs' = hs + sum_t xs_t B_t^T,
  //   e_{k+1} = e_k + c_last.
  // e_k is the incoming exponent while it stays in [|c_last| - kExpLim,
  // kExpLim]; otherwise hs is shifted by a whole number of octaves (an exact
  // ldexp) to bring e_k just below kExpLim.  A per-element sub-block shifts
  // e to within half an octave of 0 and uses
  //   y_t = 2^{c_t + e_k} hs C_t + sum_t' Score[t][t'] 2^{c_t - q_t'} x_t' + D x_t,
  //   hs' = 2^{c_last} hs + sum_t 2^{c_last - q_t - e_k} x_t B_t^T,  e_{k+1} = e_k.
  // scan() writes the per-token factors of sub-block k to slot `sl` and sets
  // the next_* scalars.
  int next_fast = 1, next_shift = 0;
  float next_clast = 0.f, next_eout = 0.f;
  auto scan = [&](int k, float rdt, float e_in, int sl) {
    const int nv = min(64, L - 64 * k);
    float dl = softplus_f(rdt + bias);
    dl = (l < nv) ? dl : 0.f;
    const float c = wave_incl_scan(dl * a2);
    float clast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c), 63));
    // Keep the (wave-uniform) decisions below in vector registers: as
    // per-lane selects they stay inside one basic block with the products
    // they are scheduled against, instead of becoming scalar branches; every
    // arm is computed before the choice so that none becomes a branch.
    float e_v = e_in;
    if constexpr (GATED)
      __asm__ volatile("" : "+v"(clast), "+v"(e_v));
    else
      __asm__("" : "+v"(clast), "+v"(e_v));
    const float q = c - hw_log2(dl); // +inf where Delta = 0
    const bool fast = fabsf(clast) <= kSpanMax;
    const bool keep = e_v >= -clast - kExpLim && e_v <= kExpLim;
    float n; // octaves
    if constexpr (GATED) {
      // (the gated walk holds the gate inputs as well; with every arm
      // computed up front it spills)
      n = fast ? (keep ? 0.f : floorf(kExpLim - e_v)) : -rintf(e_v);
    } else {
      const float n_up = floorf(kExpLim - e_v), n_fast = keep ? 0.f : n_up, n_slow = -rintf(e_v);
      n = fast ? n_fast : n_slow;
    }
    const float ek = e_v + n;
    sF0[sl][w][l] = hw_exp2((fast ? 0.f : clast) - q - ek);
    sF1[sl][w][l] = hw_exp2(c + ek);
    sQC[sl][w][l] = make_float2(q, c);
    next_fast = __builtin_amdgcn_readfirstlane((int)fast);
    next_shift = __builtin_amdgcn_readfirstlane((int)n);
    next_clast = clast;
    next_eout = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, fast ? ek + clast : ek)));
  };

  // ---- the phases of one sub-block -------------------------------------------
  // x^T fragments (row p0 + li, K = tokens), raw and scaled by the token
  // factors of slot `slot`.
  FragBF xr[2], xs[2];
  auto scale_x = [&](int slot) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      xr[ks] = trfrag(sX[w], 16, 32 * ks, 0, li, lg);
      const float4 fa = *reinterpret_cast<const float4 *>(&sF0[slot][w][32 * ks + 4 * lg]);
      const float4 fb = *reinterpret_cast<const float4 *>(&sF0[slot][w][32 * ks + 16 + 4 * lg]);
      const float v[8] = {elem(xr[ks], 0) * fa.x, elem(xr[ks], 1) * fa.y, elem(xr[ks], 2) * fa.z,
                          elem(xr[ks], 3) * fa.w, elem(xr[ks], 4) * fb.x, elem(xr[ks], 5) * fb.y,
                          elem(xr[ks], 6) * fb.z, elem(xr[ks], 7) * fb.w};
      xs[ks] = pack8<__bf16>(v);
    }
  };
  // State term Y[p][t] = sum_n hs[p][n] C[t][n]; K-step outer, the four
  // token tiles of a step are independent MFMAs read together.
  f32x4 yacc[4];
  auto state_term = [&](int slot) {
    FragBF hf[KN];
#pragma unroll
    for (int ks = 0; ks < KN; ++ks) {
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = hs[2 * ks][r];
        v[4 + r] = hs[2 * ks + 1][r];
      }
      hf[ks] = pack8<__bf16>(v);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) yacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KN; ++ks) {
      FragBF cf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) cf[u] = ld8(&sRec[slot][(ks * 4 + u) * 512 + 8 * l]);
#pragma unroll
      for (int u = 0; u < 4; ++u) yacc[u] = mma(hf[ks], cf[u], yacc[u]);
    }
  };
  // State update hs += B^T xs (after the state term has read hs).
  auto update = [&](int slot) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int kk = 0; kk < NT; ++kk) hs[kk] = mma(ld8(&sRec[slot][(NCB + ks * NT + kk) * 512 + 8 * l]), xs[ks], hs[kk]);
  };
  // Per-element path: decay the state by 2^{c_last} before its update (its xs
  // holds 2^{c_last - q - e} x).
  auto decay_state = [&](float clast) {
    const float mid = hw_exp2(clast);
#pragma unroll
    for (int kk = 0; kk < NT; ++kk) hs[kk] *= mid;
  };
  // Exact renormalisation hs *= 2^{-n}.
  auto shift_state = [&](int n) {
#pragma unroll
    for (int kk = 0; kk < NT; ++kk)
#pragma unroll
      for (int r = 0; r < 4; ++r) hs[kk][r] = __builtin_amdgcn_ldexpf(hs[kk][r], -n);
  };
  // Intra-block term added to the state term, and the token factor of y.
  auto intra = [&](int slot, auto fast_tag) {
    if constexpr (decltype(fast_tag)::value) {
      // on the shared scores; y = 2^{c + e} (state + intra)
#pragma unroll
      for (int f = 0; f < NSF; ++f) {
        const int u = f < 2 ? f : 2 + (f - 2) / 2, ks = f < 2 ? 0 : (f - 2) % 2;
        yacc[u] = mma(xs[ks], sf[f], yacc[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) yacc[u] *= sF1[slot][w][16 * u + li];
    } else {
      // per-element decay M[t][t'] = Score[t][t'] 2^{c_t - q_t'} on raw x; the
      // state term is scaled by 2^{c_t + e} first
#pragma unroll
      for (int u = 0; u < 4; ++u) yacc[u] *= sF1[slot][w][16 * u + li];
#pragma unroll
      for (int f = 0; f < NSF; ++f) {
        const int u = f < 2 ? f : 2 + (f - 2) / 2, ks = f < 2 ? 0 : (f - 2) % 2;
        const int t = 16 * u + li;
        const float ct = sQC[slot][w][t].y;
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tp = 32 * ks + kperm(lg, j);
          v[j] = (tp <= t) ? elem(sf[f], j) * hw_exp2(ct - sQC[slot][w][tp].x) : 0.f;
        }
        yacc[u] = mma(xr[ks], pack8<__bf16>(v), yacc[u]);
      }
    }
  };
  // y = acc + D x stored directly; rows past the end (and idle waves) are
  // dropped.
  const uint32_t offY = (uint32_t)((li * rowX + 4 * lg) * 2);
  __bf16 *Ybase = reinterpret_cast<__bf16 *>(prm.out) + (int64_t)ib * L * rowX + (int64_t)h * P + p0;
  // Gate input of this wave's y values of a sub-block (same positions).
  const __bf16 *Zbase = GATED ? reinterpret_cast<const __bf16 *>(prm.z) + (int64_t)ib * L * rowX + (int64_t)h * P + p0
                              : nullptr;
  float4 zq[4];
  auto fetch_z = [&](int k) {
    const int t0 = 64 * k, nv = min(64, L - t0);
    const auto rsZ = make_rsrc(Zbase + (int64_t)t0 * rowX, (uint32_t)(((int64_t)(nv - 1) * rowX + 16) * 2));
#pragma unroll
    for (int u = 0; u < 4; ++u) zq[u] = bload4x<__bf16>(rsZ, offY + (uint32_t)(16 * u * rowX * 2));
  };
  auto store_y = [&](int k) {
    const int t0 = 64 * k, nv = min(64, L - t0);
    const auto rsY = make_rsrc(Ybase + (int64_t)t0 * rowX,
                               active ? (uint32_t)(((int64_t)(nv - 1) * rowX + 16) * 2) : 0u);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(&sX[w][(16 * u + li) * 16 + 4 * lg]);
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = yacc[u][r] + d_h * (float)xv[r];
      if constexpr (GATED) {
        v[0] *= silu_f(zq[u].x);
        v[1] *= silu_f(zq[u].y);
        v[2] *= silu_f(zq[u].z);
        v[3] *= silu_f(zq[u].w);
      }
      bstore4<__bf16>(rsY, offY + (uint32_t)(16 * u * rowX * 2), v[0], v[1], v[2], v[3]);
    }
  };
  // With more than four waves: y = acc + D x of this wave's rows into the
  // workgroup tile of slot `slot`.
  auto put_y = [&](int slot) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = 16 * u + li;
      const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(&sX[w][t * 16 + 4 * lg]);
      bf16x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (__bf16)(yacc[u][r] + d_h * (float)xv[r]);
      *reinterpret_cast<bf16x4 *>(&sY[slot][t * YLD + 16 * w + 4 * lg]) = v;
    }
  };
  // Store the tile of sub-block k (after a barrier).  For one token the
  // workgroup's rows are one contiguous run of y (rows are (head, p) pairs,
  // head-major, and y is [.., token, head, p]), so the tile goes out as
  // aligned 16-byte pieces, two per thread; pieces of rows past the group's
  // last row are dropped, as are tokens past L.  k < 0 stores nothing.
  const int rows_valid = min(16 * W, prm.rows_per_bg - wi * 16 * W);
  __bf16 *Ywg = reinterpret_cast<__bf16 *>(prm.out) + (int64_t)ib * L * rowX + (int64_t)g * (H / G) * P + wi * 16 * W;
  // Gate input pieces matching the pieces flush_y stores for sub-block k
  // (zeros for k < 0).
  const __bf16 *Zwg = GATED ? reinterpret_cast<const __bf16 *>(prm.z) + (int64_t)ib * L * rowX +
                                  (int64_t)g * (H / G) * P + wi * 16 * W
                            : nullptr;
  float4 zpc[2];
  auto fetch_zpieces = [&](int k) {
    const int t0 = 64 * k, nv = min(64, L - t0);
    const auto rs = make_rsrc(Zwg + (int64_t)max(t0, 0) * rowX,
                              k >= 0 ? (uint32_t)(((int64_t)(nv - 1) * rowX + rows_valid) * 2) : 0u);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + i * NTH, t = q / (2 * W), j = q % (2 * W);
      zpc[i] = bload16(rs, 8 * j < rows_valid ? (uint32_t)((t * rowX + 8 * j) * 2) : 0xfffffff0u);
    }
  };
  auto flush_y = [&](int k) {
    const int t0 = 64 * k, nv = min(64, L - t0);
    // byte count before the select: a scalar select, not a branch (the gated
    // walk keeps the branch form, which schedules better there)
    uint32_t nbY;
    if constexpr (GATED) {
      nbY = k >= 0 ? (uint32_t)(((int64_t)(nv - 1) * rowX + rows_valid) * 2) : 0u;
    } else {
      const uint32_t nbY0 = (uint32_t)(((int64_t)(nv - 1) * rowX + rows_valid) * 2);
      nbY = k >= 0 ? nbY0 : 0u;
    }
    const auto rs = make_rsrc(Ywg + (int64_t)max(t0, 0) * rowX, nbY);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + i * NTH, t = q / (2 * W), j = q % (2 * W);
      float4 v = *reinterpret_cast<const float4 *>(&sY[k & 1][t * YLD + 8 * j]);
      if constexpr (GATED) {
        const bf16x8 yb = __builtin_bit_cast(bf16x8, v), zb = __builtin_bit_cast(bf16x8, zpc[i]);
        bf16x8 ob;
#pragma unroll
        for (int e = 0; e < 8; ++e) ob[e] = (__bf16)((float)yb[e] * silu_f((float)zb[e]));
        v = __builtin_bit_cast(float4, ob);
      }
      const uint32_t off = 8 * j < rows_valid ? (uint32_t)((t * rowX + 8 * j) * 2) : 0xfffffff0u;
      bstore16(rs, off, v);
    }
  };

  float e_final = 0.f;
  if constexpr (W <= 4) {
    // ---- one wave per SIMD: the wave's own latency sets the pace.  The
    //      factors of sub-block k are computed at its start; the state term
    //      runs first, the update last, and the renormalisation is applied
    //      unconditionally (a shift by 0 is exact) so that the block has no
    //      branch before the intra-block term.
    float rdt = fetch_dt(0);
    fetch_bcx(0);
    fetch_scores(0);
    stage(0);
    float e = 0.f;
    for (int k = 0; k < nsub; ++k) {
      const int slot = k & 1;
      lds_barrier(); // B/C/x of sub-block k staged; slot ^ 1 no longer read
      scan(k, rdt, e, slot);
      const int fast = next_fast;
      rdt = fetch_dt(k + 1);
      fetch_bcx(k + 1);
      if constexpr (GATED) fetch_z(k);
      shift_state(next_shift);
      state_term(slot);
      scale_x(slot);
      if (fast) {
        intra(slot, std::true_type{});
      } else {
        intra(slot, std::false_type{});
        decay_state(next_clast);
      }
      fetch_scores(min(k + 1, nsub - 1));
      store_y(k);
      update(slot);
      stage(slot ^ 1);
      e = next_eout;
    }
    e_final = e;
  } else {
    // ---- two waves on some SIMD: the factors of sub-block k + 1 are computed
    //      during sub-block k, next to its products, the step sizes are
    //      fetched two sub-blocks ahead, and each path (separable or
    //      per-element) is one straight block.
    float rdt_next = 0.f, rdt_next2 = 0.f;
    float cur_clast = 0.f, cur_eout = 0.f;
    auto body = [&](int k, auto fast_tag) {
      constexpr bool FAST = decltype(fast_tag)::value;
      const int slot = k & 1;
      scale_x(slot);
      state_term(slot);
      if constexpr (!FAST) decay_state(cur_clast);
      update(slot);
      flush_y(k - 1);
      scan(k + 1, rdt_next, cur_eout, slot ^ 1);
      intra(slot, fast_tag);
      fetch_scores(min(k + 1, nsub - 1));
      put_y(slot);
      stage(slot ^ 1);
    };
    fetch_bcx(0);
    const float rdt0 = fetch_dt(0);
    rdt_next = fetch_dt(1);
    fetch_scores(0);
    stage(0);
    scan(0, rdt0, 0.f, 0);
    for (int k = 0; k < nsub; ++k) {
      lds_barrier(); // B/C/x of sub-block k staged; slot ^ 1 no longer read
      fetch_bcx(k + 1);
      rdt_next2 = fetch_dt(k + 2);
      if constexpr (GATED) fetch_zpieces(k - 1);
      const int fast = next_fast;
      cur_clast = next_clast;
      cur_eout = next_eout;
      if (__builtin_expect(next_shift != 0, 0)) shift_state(next_shift);
      if (fast)
        body(k, std::true_type{});
      else
        body(k, std::false_type{});
      rdt_next = rdt_next2;
    }
    if constexpr (GATED) fetch_zpieces(nsub - 1);
    lds_barrier(); // y tile of the last sub-block complete
    flush_y(nsub - 1);
    e_final = cur_eout;
  }

  if (prm.final_state != nullptr && active) {
    const float sc = hw_exp2(e_final);
#pragma unroll
    for (int k = 0; k < NT; ++k) *reinterpret_cast<f32x4 *>(prm.final_state + srow + 16 * k + 4 * lg) = hs[k] * sc;
  }
}

template <int N, int W>
hipError_t launch_rwalk_t(const RWalkParams &p, int nwg, hipStream_t st) {
  if (p.z)
    hipLaunchKernelGGL((rwalk_kernel<N, W, true>), dim3(nwg), dim3(W * 64), 0, st, p);
  else
    hipLaunchKernelGGL((rwalk_kernel<N, W, false>), dim3(nwg), dim3(W * 64), 0, st, p);
  return hipGetLastError();
}

template <int N>
hipError_t launch_rwalk_n(int W, const RWalkParams &p, int nwg, hipStream_t st) {
  switch (W) {
  case 1: return launch_rwalk_t<N, 1>(p, nwg, st);
  case 2: return launch_rwalk_t<N, 2>(p, nwg, st);
  case 3: return launch_rwalk_t<N, 3>(p, nwg, st);
  case 4: return launch_rwalk_t<N, 4>(p, nwg, st);
  case 5: return launch_rwalk_t<N, 5>(p, nwg, st);
  case 6: return launch_rwalk_t<N, 6>(p, nwg, st);
  case 7: return launch_rwalk_t<N, 7>(p, nwg, st);
  case 8: return launch_rwalk_t<N, 8>(p, nwg, st);
  default: return hipErrorInvalidValue;
  }
}

} // namespace

hipError_t launch_rwalk(int N, int W, const RWalkParams &p, hipStream_t stream) {
  const int nwg = p.b * p.G * p.wg_per_bg;
  switch (N) {
  case 32: return launch_rwalk_n<32>(W, p, nwg, stream);
  case 64: return launch_rwalk_n<64>(W, p, nwg, stream);
  case 128: return launch_rwalk_n<128>(W, p, nwg, stream);
  default: return hipErrorInvalidValue;
  }
}

} // namespace ssd
