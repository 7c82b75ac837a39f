// ssd_prep.hip -- per (batch, group, 64-token sub-block) operand records for
// the row-sliced walk (ssd_rwalk.hip).
//
// The method ("Mamba-3 deep dive ch. 2, SSM foundations", 171host.com,
// section 2.1.2 recurrence and section 2.2.1 matrix form Y = (L o C B^T) X;
// "Transformers are SSMs" summary, gongshangzheng.github.io, section 1.2:
// quadratic form inside a block, the N-dimensional state across blocks).
// Inside a 64-token sub-block every product the walk takes has one operand
// that depends on the (batch, group) alone: C for the state term S C_t,
// B for the state update sum_t xs_t B_t^T and the raw scores C_t . B_t' for
// the intra-block term.  This kernel writes them once per (batch, group,
// sub-block), already in the per-lane order of the matrix-core fragments
// the walk feeds, so that the walk copies a record into LDS linearly and
// reads every fragment as one 16-byte, bank-conflict-free LDS read.
//
// Fragment order (v_mfma_f32_16x16x32_bf16, one 1 KiB block per fragment):
// lane l = li + 16 lg of a block holds eight bf16 K-values for row/column li
// of the fragment; the K-values of lane group lg are the positions
// {4lg .. 4lg+3, 16+4lg .. 16+4lg+3} of the 32-wide K-step (the order the
// state registers and the transposed x reads produce).
//
//   C blocks  (ks, u), ks < N/32, u < 4:   C[16u + li][32ks + K(lg)]
//   B blocks  (ks, kk), ks < 2, kk < N/16: B[32ks + K(lg)][16kk + li]
//   S blocks  (u, ks) in (0,0) (1,0) (2,0) (2,1) (3,0) (3,1):
//             S[16u + li][32ks + K(lg)], S[t][t'] = C_t . B_t' for t' <= t,
//             zero above the diagonal
//
// Tokens past the sequence end read as zero.  Record of sub-block k of
// (batch ib, group g): blocks [C | B | S] at rec + ((ib*G + g)*nsub + k) *
// rec_blocks(N) * 512 bf16.
//
// A second set of workgroups, one per (batch, sub-block), writes the step
// sizes head-major, dtT[ib][h][64k + j] (Delta = softplus(dt + dt_bias) for
// the plain walk, the raw dt for the gated walk), so that each wave of the
// walk reads its head's 64 step sizes as one contiguous 256-byte run instead
// of 64 loads 4H bytes apart; they run beside the record workgroups (two
// workgroups fit a compute unit).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kHC = 128; // heads per pass of the step-size transpose

// Head-major step sizes of sub-block k of batch ib: dtT[ib][h][64k + j] =
// softplus(dt[ib][64k + j][h] + dt_bias[h]) with `softplus`, else the raw
// dt (the raw step size read as zero past the sequence end), in
// passes of kHC heads through the LDS tile sT[head][token] (row stride 65).
// Each head's 64 step sizes are then one contiguous 256-byte run for the walk.
__device__ __forceinline__ void transpose_dt(const float *__restrict__ dt, const float *__restrict__ dt_bias,
                                             int softplus, float *__restrict__ dtT, float *sT, int ib, int k, int L,
                                             int H, int nsub, int tid) {
  const int u = tid >> 6, l = tid & 63;
  const int t0 = 64 * k, nv = min(64, L - t0), Lp = nsub * 64;
  for (int h0 = 0; h0 < H; h0 += kHC) {
    const int hc = min(kHC, H - h0);
    if (h0 > 0) __syncthreads();
    if ((H & 3) == 0) {
      // float4 pieces: lane l takes piece j of row ro of each group of rpi
      // rows (a token row of the pass holds hc / 4 pieces)
      const int H4 = hc >> 2, rpi = 64 / H4, ro = l / H4, j = l % H4;
      if (ro < rpi) {
        for (int t = u * rpi + ro; t < 64; t += 4 * rpi) {
          const float4 v = t < nv ? *reinterpret_cast<const float4 *>(dt + ((int64_t)ib * L + t0 + t) * H + h0 + 4 * j)
                                  : float4{0.f, 0.f, 0.f, 0.f};
          sT[(4 * j) * 65 + t] = v.x;
          sT[(4 * j + 1) * 65 + t] = v.y;
          sT[(4 * j + 2) * 65 + t] = v.z;
          sT[(4 * j + 3) * 65 + t] = v.w;
        }
      }
    } else {
      for (int t = u; t < 64; t += 4)
        for (int hh = l; hh < hc; hh += 64)
          sT[hh * 65 + t] = t < nv ? dt[((int64_t)ib * L + t0 + t) * H + h0 + hh] : 0.f;
    }
    __syncthreads();
    // four consecutive tokens of a head per thread (16-byte stores), as step
    // sizes Delta = softplus(dt + dt_bias), or raw when `softplus` is 0
    for (int e = tid; e < 16 * hc; e += 256) {
      const int hh = e >> 4, t = (e & 15) * 4;
      const float *r = &sT[hh * 65 + t];
      float4 v = float4{r[0], r[1], r[2], r[3]};
      if (softplus) {
        const float bias = dt_bias ? dt_bias[h0 + hh] : 0.f;
        v = float4{softplus_f(v.x + bias), softplus_f(v.y + bias), softplus_f(v.z + bias), softplus_f(v.w + bias)};
      }
      *reinterpret_cast<float4 *>(dtT + ((int64_t)ib * H + h0 + hh) * Lp + t0 + t) = v;
    }
  }
}

template <int N>
__global__ void __launch_bounds__(256) prep_kernel(const __bf16 *__restrict__ B, const __bf16 *__restrict__ C,
                                                   __bf16 *__restrict__ rec, const float *__restrict__ dt,
                                                   const float *__restrict__ dt_bias, int softplus,
                                                   float *__restrict__ dtT, int L, int H, int G, int nsub) {
  constexpr int NCB = 4 * (N / 32);     // C blocks
  constexpr int NBB = 2 * (N / 16);     // B blocks
  constexpr int NRB = NCB + NBB + 6;    // blocks per record
  constexpr int LDB = tr_ld(N, 2);      // B tile: transposed reads
  constexpr int LDC = N + 8;            // C tile: row reads
  constexpr int RW = N / 8;             // 16-byte pieces per row
  __shared__ __attribute__((aligned(16))) __bf16 sB[64 * LDB];
  __shared__ __attribute__((aligned(16))) __bf16 sC[64 * LDC];
  __shared__ float sT[kHC * 65];  // step sizes of kHC heads x 64 tokens, transposed

  const int tid = threadIdx.x, u = tid >> 6, l = tid & 63, li = l & 15, lg = l >> 4;
  const int nrec = gridDim.x - (int)(gridDim.x / (G + 1)); // b*G*nsub record workgroups
  if ((int)blockIdx.x >= nrec) {
    // the step-size workgroups, one per (batch, sub-block)
    const int wd = blockIdx.x - nrec, k = wd % nsub, ib = wd / nsub;
    transpose_dt(dt, dt_bias, softplus, dtT, sT, ib, k, L, H, nsub, tid);
    return;
  }
  const int wg = blockIdx.x;
  const int k = wg % nsub, bg = wg / nsub;
  const int g = bg % G, ib = bg / G;
  const int t0 = 64 * k, nv = min(64, L - t0);
  const int64_t rowB = (int64_t)G * N;
  const int64_t base = ((int64_t)ib * L + t0) * rowB + (int64_t)g * N;
  const uint32_t bytes = (uint32_t)(((int64_t)(nv - 1) * rowB + N) * 2);
  const auto rsB = make_rsrc(B + base, bytes);
  const auto rsC = make_rsrc(C + base, bytes);
  for (int q = tid; q < 64 * RW; q += 256) {
    const int j = q / RW, n0 = (q % RW) * 8;
    const uint32_t off = (uint32_t)((j * rowB + n0) * 2);
    *reinterpret_cast<float4 *>(&sB[j * LDB + n0]) = bload16(rsB, off);
    *reinterpret_cast<float4 *>(&sC[j * LDC + n0]) = bload16(rsC, off);
  }
  __syncthreads();

  __bf16 *out = rec + ((int64_t)bg * nsub + k) * (NRB * 512);
  // C blocks: wave u writes the blocks of token tile u
#pragma unroll
  for (int ks = 0; ks < N / 32; ++ks) {
    const FragBF f = ld4x2(&sC[(16 * u + li) * LDC + 32 * ks + 4 * lg], &sC[(16 * u + li) * LDC + 32 * ks + 16 + 4 * lg]);
    *reinterpret_cast<bf16x8 *>(out + (ks * 4 + u) * 512 + 8 * l) = f.v;
  }
  // B blocks: transposed reads of the B tile, blocks split over the waves
  for (int blk = u; blk < NBB; blk += 4) {
    const int ks = blk / (N / 16), kk = blk % (N / 16);
    const FragBF f = trfrag(sB, LDB, 32 * ks, 16 * kk, li, lg);
    *reinterpret_cast<bf16x8 *>(out + (NCB + blk) * 512 + 8 * l) = f.v;
  }
  // Scores of query tile u: A operand = C rows of the queries (K = n),
  // B operand = B rows of the keys; D[t][t'] in the accumulator layout
  // (rows 4lg + r = t' within the key tile, column li = t within tile u).
  FragBF cq[N / 32];
#pragma unroll
  for (int ks = 0; ks < N / 32; ++ks) cq[ks] = ld8(&sC[(16 * u + li) * LDC + 32 * ks + 8 * lg]);
  // key tiles 0..u; a key tile jt supplies K-values of the score fragment
  // (u, jt / 2): positions 4lg + r (jt even) or 16 + 4lg + r (jt odd)
  float sv[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[a][e] = 0.f;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    if (jt > u) break;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks)
      acc = mma(ld8(&sB[(16 * jt + li) * LDB + 32 * ks + 8 * lg]), cq[ks], acc);
    // acc[r] = B_{16jt + 4lg + r} . C_{16u + li} = S[16u + li][16jt + 4lg + r]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool keep = 16 * jt + 4 * lg + r <= 16 * u + li;
      sv[jt / 2][4 * (jt % 2) + r] = keep ? acc[r] : 0.f;
    }
  }
  // score blocks of tile u: (u, 0) and, for u >= 2, (u, 1)
  const int sb0 = u < 2 ? u : 2 + 2 * (u - 2);
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    if (a == 1 && u < 2) break;
    *reinterpret_cast<bf16x8 *>(out + (NCB + NBB + sb0 + a) * 512 + 8 * l) = pack8<__bf16>(sv[a]).v;
  }
}

} // namespace

int prep_record_blocks(int N) { return 4 * (N / 32) + 2 * (N / 16) + 6; }

hipError_t launch_prep(const void *B, const void *C, void *rec, const float *dt, const float *dt_bias, int softplus,
                       float *dtT, int b, int L, int H, int G, int N, hipStream_t stream) {
  const int nsub = (L + 63) / 64;
  // b*G*nsub record workgroups, then b*nsub step-size workgroups
  const dim3 grid((unsigned)(b * G * nsub + b * nsub));
  const __bf16 *Bp = reinterpret_cast<const __bf16 *>(B);
  const __bf16 *Cp = reinterpret_cast<const __bf16 *>(C);
  __bf16 *r = reinterpret_cast<__bf16 *>(rec);
  switch (N) {
  case 32: hipLaunchKernelGGL(prep_kernel<32>, grid, dim3(256), 0, stream, Bp, Cp, r, dt, dt_bias, softplus, dtT, L, H, G, nsub); break;
  case 64: hipLaunchKernelGGL(prep_kernel<64>, grid, dim3(256), 0, stream, Bp, Cp, r, dt, dt_bias, softplus, dtT, L, H, G, nsub); break;
  case 128: hipLaunchKernelGGL(prep_kernel<128>, grid, dim3(256), 0, stream, Bp, Cp, r, dt, dt_bias, softplus, dtT, L, H, G, nsub); break;
  default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

} // namespace ssd
