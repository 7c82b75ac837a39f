// ssd_sscan.hip -- selective scan with a per-channel step size and a
// diagonal A per (channel, state index), on MI355X (gfx950).
//
// The operation is the Mamba-1 selective SSM (Mamba paper-reading notes,
// sxlin0.github.io, the selective-mechanism section: B, C and Delta depend
// on the input, Delta = softplus(parameter + s_Delta(x)) per channel; the
// "Transformers are SSMs" summary, gongshangzheng.github.io, section 1.3
// table: Mamba-1 keeps a small state, N = 16).  For every batch row and
// channel d:
//
//     Delta_t = softplus(dt[t][d] + dt_bias[d])
//     h_t[n]  = exp(Delta_t A[d][n]) h_{t-1}[n] + Delta_t B_t[n] x_t[d]
//     y_t[d]  = sum_n C_t[n] h_t[n] + D[d] x_t[d]
//
// Layout of the work.  One wave owns 64 consecutive channels of one batch
// row (lane = channel, its N states in registers) over one segment of the
// sequence.  The 64 channels read one B/C group, so B_t and C_t are the
// same for the whole wave and are fetched with wave-uniform loads.  Each
// (token, channel) costs N exponentials, so the scan is bound by the vector
// ALU, not by HBM; the sequence is cut into segments to give every SIMD
// several waves:
//
//   pass 0 (segments 0 .. nseg-2): the segment's end state from a zero
//          state (segment 0: from the initial state, which it also copies
//          to scratch) and the segment's sum of Delta;
//   pass 1 (every segment): the entering state folded from pass 0's
//          results, h = exp(A sum Delta_q) h + h_end_q over the earlier
//          segments, then the recurrence with outputs; the last segment
//          writes the final state.
//
// Only pass 0 reads the initial state, so the final state may alias it.
#include "ssd_device.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kTok = 8; // tokens per unrolled step (and granule of segments)

template <typename T> __device__ __forceinline__ float ld_elem(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ float ld_elem<__bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const uint16_t u = __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
  return __builtin_bit_cast(float, (uint32_t)u << 16);
}
template <> __device__ __forceinline__ float ld_elem<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return bload4(r, off);
}
template <typename T> __device__ __forceinline__ void st_elem(__amdgpu_buffer_rsrc_t r, uint32_t off, float v);
template <> __device__ __forceinline__ void st_elem<__bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  const __bf16 b = (__bf16)v;
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, b), r, (int)off, 0, 0);
}
template <> __device__ __forceinline__ void st_elem<float>(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r, (int)off, 0, 0);
}

// N consecutive values at a wave-uniform address, read through the scalar
// unit (constant address space: B and C are not written while the kernel
// runs), widened to fp32.
template <typename T, int N> __device__ __forceinline__ void load_uniform(const T *p, float *v);
template <int N> __device__ __forceinline__ void load_uniform_bf16(const __bf16 *p, float *v) {
  typedef __attribute__((address_space(4))) const uint32_t *cptr;
  const cptr q = (cptr)p;
#pragma unroll
  for (int i = 0; i < N / 2; ++i) {
    const uint32_t w = q[i];
    v[2 * i] = __builtin_bit_cast(float, w << 16);
    v[2 * i + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void load_uniform<__bf16, 4>(const __bf16 *p, float *v) { load_uniform_bf16<4>(p, v); }
template <> __device__ __forceinline__ void load_uniform<__bf16, 8>(const __bf16 *p, float *v) { load_uniform_bf16<8>(p, v); }
template <> __device__ __forceinline__ void load_uniform<__bf16, 16>(const __bf16 *p, float *v) { load_uniform_bf16<16>(p, v); }
template <int N> __device__ __forceinline__ void load_uniform_f32(const float *p, float *v) {
  typedef __attribute__((address_space(4))) const float *cptr;
  const cptr q = (cptr)p;
#pragma unroll
  for (int i = 0; i < N; ++i) v[i] = q[i];
}
template <> __device__ __forceinline__ void load_uniform<float, 4>(const float *p, float *v) { load_uniform_f32<4>(p, v); }
template <> __device__ __forceinline__ void load_uniform<float, 8>(const float *p, float *v) { load_uniform_f32<8>(p, v); }
template <> __device__ __forceinline__ void load_uniform<float, 16>(const float *p, float *v) { load_uniform_f32<16>(p, v); }

template <typename T, int N, int PASS>
__global__ void __launch_bounds__(64) sscan_kernel(const SScanParams p, const T *__restrict__ Bp,
                                                   const T *__restrict__ Cp) {
  const int Dc = p.Dc, L = p.L, nseg = p.nseg, cgroups = Dc / 64;
  const int wg = blockIdx.x;
  const int seg = wg % nseg, cg = (wg / nseg) % cgroups, ib = wg / (nseg * cgroups);
  if (PASS == 0 && seg == nseg - 1) return; // nothing reads the last end state
  const int l = threadIdx.x;
  const int d = cg * 64 + l;
  const int g = (int)(((int64_t)cg * 64 * p.G) / Dc); // the wave's group
  const int t_begin = seg * p.seg_len, t_end = min(L, t_begin + p.seg_len);
  const int nt = t_end - t_begin;

  float a2[N]; // A * log2(e): the gate is exp2(Delta * a2)
#pragma unroll
  for (int n = 0; n < N; ++n) a2[n] = p.A[(int64_t)d * N + n] * kLog2e;
  const float bias = p.dt_bias ? p.dt_bias[d] : 0.f;
  const float dd = p.D ? p.D[d] : 0.f;

  const int64_t bd = (int64_t)ib * Dc + d;
  float h[N];
  if (PASS == 0) {
    if (seg == 0 && p.init) {
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = p.init[bd * N + n];
#pragma unroll
      for (int n = 0; n < N; ++n) p.hcopy[bd * N + n] = h[n];
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = 0.f;
    }
  } else if (nseg == 1) {
#pragma unroll
    for (int n = 0; n < N; ++n) h[n] = p.init ? p.init[bd * N + n] : 0.f;
  } else {
    // entering state: segment 0 from the staged initial state, later
    // segments folded from pass 0's end states
    const int64_t sd = (int64_t)ib * nseg * Dc + d; // (ib, q = 0, d)
    if (seg == 0) {
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = p.init ? p.hcopy[bd * N + n] : 0.f;
    } else {
#pragma unroll
      for (int n = 0; n < N; ++n) h[n] = p.hend[sd * N + n];
      // the end states of the earlier segments four at a time: the loads
      // of a group are issued together, then folded in order
      for (int q0 = 1; q0 < seg; q0 += 4) {
        float hb[4][N], sb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t sq = sd + (int64_t)min(q0 + j, seg - 1) * Dc;
          sb[j] = p.sdelta[sq];
#pragma unroll
          for (int n = 0; n < N; ++n) hb[j][n] = p.hend[sq * N + n];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (q0 + j >= seg) break;
#pragma unroll
          for (int n = 0; n < N; ++n) h[n] = hw_exp2(a2[n] * sb[j]) * h[n] + hb[j][n];
        }
      }
    }
  }

  // x, dt and y of this wave over the segment: token t, lane l at byte
  // offset (t * Dc + l) * size (rows past the segment read as zero)
  const int64_t row0 = ((int64_t)ib * L + t_begin) * Dc + cg * 64;
  const uint32_t span = nt > 0 ? (uint32_t)((int64_t)(nt - 1) * Dc + 64) : 0u;
  const auto rsX = make_rsrc(reinterpret_cast<const T *>(p.x) + row0, span * (uint32_t)sizeof(T));
  const auto rsD = make_rsrc(p.dt + row0, span * 4u);
  const auto rsY = make_rsrc(reinterpret_cast<T *>(p.out) + row0, span * (uint32_t)sizeof(T));
  const int64_t rowBC = (int64_t)p.G * N;
  const T *Bw = Bp + ((int64_t)ib * L + t_begin) * rowBC + (int64_t)g * N;
  const T *Cw = Cp + ((int64_t)ib * L + t_begin) * rowBC + (int64_t)g * N;

  float xr[kTok], dr[kTok];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      const uint32_t o = (uint32_t)((t0 + u) * Dc + l);
      xr[u] = ld_elem<T>(rsX, o * (uint32_t)sizeof(T));
      dr[u] = bload4(rsD, o * 4u);
    }
  };
  float dsum = 0.f;
  fetch(0);
  for (int t0 = 0; t0 < nt; t0 += kTok) {
    float xc[kTok], dc[kTok];
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      xc[u] = xr[u];
      dc[u] = dr[u];
    }
    fetch(t0 + kTok);
#pragma unroll
    for (int u = 0; u < kTok; ++u) {
      const int t = t0 + u;
      if (t >= nt) break;
      // B_t and C_t: the same N values for the whole wave
      const int64_t o = (int64_t)t * rowBC;
      float bv[N], cv[N];
      load_uniform<T, N>(Bw + o, bv);
      load_uniform<T, N>(Cw + o, cv);
      const float dl = softplus_f(dc[u] + bias);
      const float dx = dl * xc[u];
      float acc = 0.f;
#pragma unroll
      for (int n = 0; n < N; ++n) {
        h[n] = hw_exp2(dl * a2[n]) * h[n] + dx * bv[n];
        acc += cv[n] * h[n];
      }
      if (PASS == 1)
        st_elem<T>(rsY, (uint32_t)(t * Dc + l) * (uint32_t)sizeof(T), acc + dd * xc[u]);
      else
        dsum += dl;
    }
  }

  if (PASS == 0) {
    const int64_t sq = ((int64_t)ib * nseg + seg) * Dc + d;
#pragma unroll
    for (int n = 0; n < N; ++n) p.hend[sq * N + n] = h[n];
    p.sdelta[sq] = dsum;
  } else if (seg == nseg - 1 && p.final_state) {
#pragma unroll
    for (int n = 0; n < N; ++n) p.final_state[bd * N + n] = h[n];
  }
}

template <typename T, int N>
hipError_t launch_sscan_t(const SScanParams &p, hipStream_t st) {
  const int grid = p.b * (p.Dc / 64) * p.nseg;
  if (p.nseg > 1) {
    hipLaunchKernelGGL((sscan_kernel<T, N, 0>), dim3(grid), dim3(64), 0, st, p,
                       reinterpret_cast<const T *>(p.B), reinterpret_cast<const T *>(p.C));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((sscan_kernel<T, N, 1>), dim3(grid), dim3(64), 0, st, p,
                     reinterpret_cast<const T *>(p.B), reinterpret_cast<const T *>(p.C));
  return hipGetLastError();
}

} // namespace

hipError_t launch_sscan(int dtype, int N, const SScanParams &p, hipStream_t st) {
  if (dtype == 1) {
    switch (N) {
    case 4: return launch_sscan_t<__bf16, 4>(p, st);
    case 8: return launch_sscan_t<__bf16, 8>(p, st);
    case 16: return launch_sscan_t<__bf16, 16>(p, st);
    }
  } else {
    switch (N) {
    case 4: return launch_sscan_t<float, 4>(p, st);
    case 8: return launch_sscan_t<float, 8>(p, st);
    case 16: return launch_sscan_t<float, 16>(p, st);
    }
  }
  return hipErrorInvalidValue;
}

} // namespace ssd
