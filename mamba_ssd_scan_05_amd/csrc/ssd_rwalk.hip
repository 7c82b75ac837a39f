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
// sub-blocks.  A sub-block's whole record (C, B and score fragments) is
// copied once into LDS and read by every wave (one 16-byte read per
// fragment); each wave holds its 16 x N state in MFMA accumulator
// registers and has its own 16 columns of x copied into a private LDS tile.
// The copies go straight from global memory to LDS (buffer loads to LDS),
// one sub-block ahead, so they hold no registers; the decay factors of the
// next sub-block are formed next to the current sub-block's state update.
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
  constexpr int NT = N / 16;             // n-tiles of the state
  constexpr int KN = N / 32;             // K-steps over n
  constexpr int NCB = 4 * KN;            // C fragment blocks of a record
  constexpr int NBB = 2 * NT;            // B fragment blocks of a record
  constexpr int NRB = NCB + NBB + 6;     // blocks per record (C, B, scores)
  constexpr int NSF = 6;                 // score fragments per sub-block

  // A sub-block's record and each wave's x tile are copied from global
  // memory straight into LDS (buffer loads to LDS: no registers, no LDS
  // writes), double-buffered.  The two buffers are distinct arrays and the
  // loop is unrolled by two, so every LDS address is static: the compiler
  // can tell the buffer being read from the one being filled and adds no
  // wait for the copy in flight.
  __shared__ __attribute__((aligned(16))) __bf16 sRecA[NRB * 512];
  __shared__ __attribute__((aligned(16))) __bf16 sRecB[NRB * 512];
  __shared__ __attribute__((aligned(16))) __bf16 sXA[W][64 * 16]; // x[token][16 columns]
  __shared__ __attribute__((aligned(16))) __bf16 sXB[W][64 * 16];
  // per-wave token factors, two sub-blocks: those of sub-block k + 1 are
  // formed at the end of sub-block k, next to its state update
  __shared__ __attribute__((aligned(16))) float sF0[2][W][64];  // xs scale (fast) / w (slow)
  __shared__ __attribute__((aligned(16))) float sF1[2][W][64];  // y scale 2^{c + e}
  __shared__ __attribute__((aligned(16))) float2 sQC[2][W][64]; // (q, c) for the slow path

  const int H = prm.H, G = prm.G, L = prm.L, P = prm.P;
  const int nwg = gridDim.x, bid = blockIdx.x;
  // XCD-aware order: consecutive ids go round-robin to the 8 XCDs; give
  // each XCD a contiguous range of logical ids so that the workgroups of one
  // (batch, group) share its records through one L2.
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
  const int nsub = (L + 63) / 64;
  // step sizes of this head, head-major (written by prep_kernel): Delta =
  // softplus(dt + dt_bias) for the plain walk, the raw dt for the gated one,
  // which applies the softplus itself (measured faster there)
  const float *dtbase = prm.dtT + ((int64_t)ib * H + h) * (nsub * 64);
  // records of this (batch, group), one per sub-block
  const __bf16 *Rbase = reinterpret_cast<const __bf16 *>(prm.rec) + (int64_t)bg * nsub * (NRB * 512);

  // x pieces of this wave: piece l + 64e = (token, half) -> 8 columns, which
  // lands at byte 16 (l + 64e) of the wave's x tile (one 1 KiB copy per e).
  uint32_t offX[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int pc = l + 64 * e, tok = pc >> 1, half = pc & 1;
    offX[e] = (uint32_t)((tok * rowX + 8 * half) * 2);
  }
  // Copy the record and the x tiles of sub-block k into (rec, xt).  The
  // copying waves (WC of them) take record blocks w, w + WC, ... (the last
  // block again where a wave has none of its own, so they issue the same
  // number of record copies); copies past the end of the sequence use empty
  // ranges and write zeros.  With five waves the fifth shares a SIMD with
  // the first and loses issue priority to it, so it is the last to reach
  // each barrier: it issues no copies (each copy instruction holds its wave
  // for a while), waves 0-3 copy the whole record and waves 1 and 2 one half
  // each of its x tile besides their own.
  constexpr bool kSpare4 = (W == 5);
  constexpr int WC = kSpare4 ? 4 : W;
  constexpr int CPW = (NRB + WC - 1) / WC; // record blocks per copying wave
  const __bf16 *Xbase4 = nullptr;          // x columns of wave 4
  if constexpr (kSpare4) {
    const int R4 = (wi * W + 4) * 16, Rc4 = R4 < prm.rows_per_bg ? R4 : 0;
    Xbase4 = reinterpret_cast<const __bf16 *>(prm.x) + (int64_t)ib * L * rowX + (int64_t)(g * (H / G) + Rc4 / P) * P +
             Rc4 % P;
  }
  auto copy_in = [&](int k, __bf16 *rec, __bf16 (*xt)[1024]) {
    const int t0 = 64 * k, nv = min(64, L - t0);
    const auto rsR = make_rsrc(Rbase + (int64_t)min(k, nsub - 1) * (NRB * 512), nv > 0 ? (uint32_t)NRB * 1024u : 0u);
    const uint32_t xbytes = nv > 0 ? (uint32_t)(((int64_t)(nv - 1) * rowX + 16) * 2) : 0u;
    if (!kSpare4 || w < 4) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        int c = min(w + i * WC, NRB - 1);
        if constexpr (kSpare4 && !GATED) {
          // wave 0 (sharing its SIMD with wave 4) leaves its last two blocks
          // to waves 2 and 3, whose last slots pass the end of the record
          // (NRB = 2 mod 4); measured slower for the gated walk, which keeps
          // the duplicate copies
          if (w == 0 && i >= CPW - 2) continue;
          if (w + i * WC >= NRB) c = 4 * (CPW - 2) + 4 * (w - 2);
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsR, (__attribute__((address_space(3))) void *)&rec[c * 512], 16,
                                                 l * 16, c * 1024, 0, 0);
      }
      const auto rsX = make_rsrc(Xbase + (int64_t)t0 * rowX, xbytes);
#pragma unroll
      for (int e = 0; e < 2; ++e)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsX, (__attribute__((address_space(3))) void *)&xt[w][512 * e], 16,
                                                 offX[e], 0, 0, 0);
    }
    if constexpr (kSpare4) {
      if (w == 1 || w == 2) {
        const int e = w - 1;
        const auto rsX4 = make_rsrc(Xbase4 + (int64_t)t0 * rowX, xbytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsX4, (__attribute__((address_space(3))) void *)&xt[4][512 * e], 16,
                                                 offX[e], 0, 0, 0);
      }
    }
  };
  // Step size of token l of sub-block k (Delta; the raw dt for the gated
  // walk): one contiguous 256-byte run per wave, nothing read for k past the
  // last sub-block.
  auto fetch_dt = [&](int k) {
    const auto rsD = make_rsrc(dtbase + 64 * (int64_t)min(k, nsub - 1), k < nsub ? 256u : 0u);
    return bload4(rsD, (uint32_t)(l * 4));
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
  // scan() writes the per-token factors of sub-block k and sets the next_*
  // scalars.
  int next_fast = 1, next_shift = 0;
  float next_clast = 0.f, next_eout = 0.f;
  auto scan = [&](int k, float rdt, float e_in, int fs) {
    const int nv = min(64, L - 64 * k);
    float dl;
    if constexpr (GATED) {
      dl = softplus_f(rdt + bias);
      dl = (l < nv) ? dl : 0.f;
    } else {
      dl = (l < nv) ? rdt : 0.f;
    }
    const float c = wave_incl_scan(dl * a2);
    float clast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, c), 63));
    // Keep the (wave-uniform) decisions below in vector registers: as
    // per-lane selects they stay inside one basic block with the products
    // they are scheduled against, instead of becoming scalar branches.
    float e_v = e_in;
    __asm__("" : "+v"(clast), "+v"(e_v));
    const float q = c - hw_log2(dl); // +inf where Delta = 0
    const bool fast = fabsf(clast) <= kSpanMax;
    const bool keep = e_v >= -clast - kExpLim && e_v <= kExpLim;
    const float n_up = floorf(kExpLim - e_v), n_fast = keep ? 0.f : n_up, n_slow = -rintf(e_v);
    const float n = fast ? n_fast : n_slow; // octaves
    const float ek = e_v + n;
    sF0[fs][w][l] = hw_exp2((fast ? 0.f : clast) - q - ek);
    sF1[fs][w][l] = hw_exp2(c + ek);
    sQC[fs][w][l] = make_float2(q, c);
    next_fast = __builtin_amdgcn_readfirstlane((int)fast);
    next_shift = __builtin_amdgcn_readfirstlane((int)n);
    next_clast = clast;
    next_eout = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, fast ? ek + clast : ek)));
  };

  // ---- the phases of one sub-block -------------------------------------------
  // x^T fragments (row p0 + li, K = tokens) scaled by the token factors.
  FragBF xs[2];
  auto scale_x = [&](const __bf16 (*xt)[1024], int fs) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const FragBF xr = trfrag(xt[w], 16, 32 * ks, 0, li, lg);
      const float4 fa = *reinterpret_cast<const float4 *>(&sF0[fs][w][32 * ks + 4 * lg]);
      const float4 fb = *reinterpret_cast<const float4 *>(&sF0[fs][w][32 * ks + 16 + 4 * lg]);
      const float v[8] = {elem(xr, 0) * fa.x, elem(xr, 1) * fa.y, elem(xr, 2) * fa.z, elem(xr, 3) * fa.w,
                          elem(xr, 4) * fb.x, elem(xr, 5) * fb.y, elem(xr, 6) * fb.z, elem(xr, 7) * fb.w};
      xs[ks] = pack8<__bf16>(v);
    }
  };
  // State term Y[p][t] = sum_n hs[p][n] C[t][n]; K-step outer, the four
  // token tiles of a step are independent MFMAs.
  f32x4 yacc[4];
  auto state_term = [&](const __bf16 *rec) {
#pragma unroll
    for (int u = 0; u < 4; ++u) yacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KN; ++ks) {
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = hs[2 * ks][r];
        v[4 + r] = hs[2 * ks + 1][r];
      }
      const FragBF hf = pack8<__bf16>(v);
#pragma unroll
      for (int u = 0; u < 4; ++u) yacc[u] = mma(hf, ld8(&rec[(ks * 4 + u) * 512 + 8 * l]), yacc[u]);
    }
  };
  // State update hs += B^T xs (after the state term has read hs).
  auto update = [&](const __bf16 *rec) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int kk = 0; kk < NT; ++kk) hs[kk] = mma(ld8(&rec[(NCB + ks * NT + kk) * 512 + 8 * l]), xs[ks], hs[kk]);
  };
  // Intra-block term added to the state term, and the token factor of y.
  auto intra = [&](const __bf16 *rec, const __bf16 (*xt)[1024], int fs, auto fast_tag) {
    if constexpr (decltype(fast_tag)::value) {
      // on the shared scores; y = 2^{c + e} (state + intra)
#pragma unroll
      for (int f = 0; f < NSF; ++f) {
        const int u = f < 2 ? f : 2 + (f - 2) / 2, ks = f < 2 ? 0 : (f - 2) % 2;
        yacc[u] = mma(xs[ks], ld8(&rec[(NCB + NBB + f) * 512 + 8 * l]), yacc[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) yacc[u] *= sF1[fs][w][16 * u + li];
    } else {
      // per-element decay M[t][t'] = Score[t][t'] 2^{c_t - q_t'} on raw x; the
      // state term is scaled by 2^{c_t + e} first
#pragma unroll
      for (int u = 0; u < 4; ++u) yacc[u] *= sF1[fs][w][16 * u + li];
#pragma unroll
      for (int f = 0; f < NSF; ++f) {
        const int u = f < 2 ? f : 2 + (f - 2) / 2, ks = f < 2 ? 0 : (f - 2) % 2;
        const int t = 16 * u + li;
        const float ct = sQC[fs][w][t].y;
        const FragBF sfr = ld8(&rec[(NCB + NBB + f) * 512 + 8 * l]);
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tp = 32 * ks + kperm(lg, j);
          v[j] = (tp <= t) ? elem(sfr, j) * hw_exp2(ct - sQC[fs][w][tp].x) : 0.f;
        }
        yacc[u] = mma(trfrag(xt[w], 16, 32 * ks, 0, li, lg), pack8<__bf16>(v), yacc[u]);
      }
    }
  };
  // y = acc + D x stored directly (times silu(z) when gated); rows past the
  // end (and idle waves) are dropped by the range check.
  const uint32_t offY = (uint32_t)((li * rowX + 4 * lg) * 2);
  __bf16 *Ybase = reinterpret_cast<__bf16 *>(prm.out) + (int64_t)ib * L * rowX + (int64_t)h * P + p0;
  const __bf16 *Zbase = GATED ? reinterpret_cast<const __bf16 *>(prm.z) + (int64_t)ib * L * rowX + (int64_t)h * P + p0
                              : nullptr;
  // z of the current sub-block (zq) and of the next one (zn, loaded a
  // sub-block ahead so that its latency is hidden behind a whole sub-block)
  bf16x4 zq[4], zn[4];
  auto fetch_z = [&](int k) {
    const int t0 = 64 * k, nv = min(64, L - t0);
    const auto rsZ = make_rsrc(Zbase + (int64_t)t0 * rowX, nv > 0 ? (uint32_t)(((int64_t)(nv - 1) * rowX + 16) * 2) : 0u);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      zn[u] = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(rsZ, (int)(offY + (uint32_t)(16 * u * rowX * 2)), 0, 0));
  };
  auto store_y = [&](int k, const __bf16 (*xt)[1024]) {
    const int t0 = 64 * k, nv = min(64, L - t0);
    const auto rsY = make_rsrc(Ybase + (int64_t)t0 * rowX,
                               active ? (uint32_t)(((int64_t)(nv - 1) * rowX + 16) * 2) : 0u);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const bf16x4 xv = *reinterpret_cast<const bf16x4 *>(&xt[w][(16 * u + li) * 16 + 4 * lg]);
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = yacc[u][r] + d_h * (float)xv[r];
      if constexpr (GATED) {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] *= silu_f((float)zq[u][r]);
      }
      bstore4<__bf16>(rsY, offY + (uint32_t)(16 * u * rowX * 2), v[0], v[1], v[2], v[3]);
    }
  };

  // ---- the walk ------------------------------------------------------------
  // Per sub-block k: barrier (the copies of k have landed, every wave is done
  // with the other buffer), the copies of k + 1 into the other buffer, the
  // state term, the intra term, y, the state update, and the factors of
  // sub-block k + 1 (their step sizes were fetched one sub-block earlier), so
  // that their scan chain runs next to the update's products.  The four y
  // stores are the last memory operations of a sub-block (loads cannot move
  // past them); the barrier waits for everything older (vmcnt(4)).
  float rdt = fetch_dt(0);
  copy_in(0, sRecA, sXA);
  if constexpr (GATED) fetch_z(0);
  __builtin_amdgcn_s_waitcnt(0x70); // vmcnt(0) expcnt(7) lgkmcnt(0)
  scan(0, rdt, 0.f, 0);
  rdt = fetch_dt(1);
  int cur_fast = next_fast, cur_shift = next_shift;
  float cur_clast = next_clast, e = next_eout;
  auto step = [&](int k, const __bf16 *rec, __bf16 (*xt)[1024], __bf16 *recN, __bf16 (*xtN)[1024]) {
    const int fs = k & 1;
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x74); // vmcnt(4) expcnt(7) lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    copy_in(k + 1, recN, xtN);
    const float rdt_next = fetch_dt(k + 2);
    if constexpr (GATED) {
#pragma unroll
      for (int u = 0; u < 4; ++u) zq[u] = zn[u];
      fetch_z(k + 1);
    }
    if (cur_shift != 0) {
#pragma unroll
      for (int kk = 0; kk < NT; ++kk)
#pragma unroll
        for (int r = 0; r < 4; ++r) hs[kk][r] = __builtin_amdgcn_ldexpf(hs[kk][r], -cur_shift);
    }
    state_term(rec);
    scale_x(xt, fs);
    if (cur_fast) {
      intra(rec, xt, fs, std::true_type{});
    } else {
      intra(rec, xt, fs, std::false_type{});
      const float mid = hw_exp2(cur_clast);
#pragma unroll
      for (int kk = 0; kk < NT; ++kk) hs[kk] *= mid;
    }
    store_y(k, xt);
    update(rec);
    // the factors of sub-block k + 1 (rdt holds its step sizes)
    scan(k + 1, rdt, e, fs ^ 1);
    cur_fast = next_fast;
    cur_shift = next_shift;
    cur_clast = next_clast;
    e = next_eout;
    rdt = rdt_next;
  };
  for (int k = 0; k < nsub; k += 2) {
    step(k, sRecA, sXA, sRecB, sXB);
    if (k + 1 < nsub) step(k + 1, sRecB, sXB, sRecA, sXA);
  }
  // e now holds the exponent after the last sub-block: scan(nsub) of an empty
  // sub-block (Delta = 0, no decay) keeps it unless it renormalises; undo that
  // renormalisation's shift, which hs never received
  e -= (float)cur_shift;

  if (prm.final_state != nullptr && active) {
    const float sc = hw_exp2(e);
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
