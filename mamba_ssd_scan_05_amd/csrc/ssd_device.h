// ssd_device.h -- device helpers shared by the gfx950 kernels of libssd:
// MFMA fragment types and loads, LDS transposed reads, raw buffer access,
// hardware exp2/log2, softplus and a wave-wide prefix sum.
//
// Fragment convention for a 16x16 tile and one K-step of 32: lane l supplies
// row/column (l % 16) and eight K-values selected by the lane group l / 16;
// the A and B operands use the same K selection, so the K order inside a
// step is free.  The accumulator holds D[4*(l/16) + r][l % 16], r = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Hardware base-2 exponential and logarithm (v_exp_f32, v_log_f32).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }

// silu(v) = v / (1 + e^{-v}); for v far below 0 the exponential is +inf
// and the result a signed zero.
__device__ __forceinline__ float silu_f(float v) {
  return v * __builtin_amdgcn_rcpf(1.f + hw_exp2(-v * kLog2e));
}

// softplus(z) = log(1 + e^z) = max(z, 0) + log1p(u), u = e^{-|z|} in (0, 1].
// log1p(u) = log(w) * u / (w - 1) with w = fl(1 + u) cancels the rounding of
// 1 + u (the classic accurate-log1p identity); w == 1 means log1p(u) = u to
// working precision.
__device__ __forceinline__ float softplus_f(float z) {
  const float u = hw_exp2(-fabsf(z) * kLog2e);
  const float w = 1.f + u;
  const float lp = (w == 1.f) ? u : hw_log2(w) * kLn2 * (u * __builtin_amdgcn_rcpf(w - 1.f));
  return fmaxf(z, 0.f) + lp;
}

// Raw buffer access: reads past `bytes` return zero and writes past it are
// dropped by the hardware range check.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
// Store 16 bytes at byte offset `off` (dropped past the range).
__device__ __forceinline__ void bstore16(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)off, 0, 0);
}
// Streaming variants for data touched once (the non-temporal cache-policy
// bit of the buffer access): keeps a stream that is read once and written
// once from displacing reused lines.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ float4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kNonTemporal));
}
__device__ __forceinline__ void bstore16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)off, 0, kNonTemporal);
}
// Load four consecutive elements of type T at byte offset `off` as floats
// (zeros past the range).
template <typename T> __device__ __forceinline__ float4 bload4x(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <> __device__ __forceinline__ float4 bload4x<__bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const bf16x4 v = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
  return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}
template <> __device__ __forceinline__ float4 bload4x<float>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return bload16(r, off);
}
// Store four outputs (converted to T) at byte offset `off`.
template <typename T> __device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, uint32_t off, float a, float b, float c, float d);
template <> __device__ __forceinline__ void bstore4<__bf16>(__amdgpu_buffer_rsrc_t r, uint32_t off, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, v), r, (int)off, 0, 0);
}
template <> __device__ __forceinline__ void bstore4<float>(__amdgpu_buffer_rsrc_t r, uint32_t off, float a, float b, float c, float d) {
  const float4 v = make_float4(a, b, c, d);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, v), r, (int)off, 0, 0);
}

// Transposed read of a row-major LDS tile: within each 16-lane group, lane li
// receives column col0 + li of rows row0 .. row0+3 (gfx950
// ds_read_b64_tr_b16; lane 4r+s of the group supplies the address of row r,
// columns 4s .. 4s+3).
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 lds_bf16x4;
__device__ __forceinline__ bf16x4 tr4(const __bf16 *tile, int ld, int row0, int col0, int li) {
  const __bf16 *p = tile + (row0 + (li >> 2)) * ld + col0 + 4 * (li & 3);
  auto q = (__attribute__((address_space(3))) lds_bf16x4 *)(p);
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(q));
}
// Fragment of eight K-values along the rows (tokens) of a row-major tile for
// column col0 + li: rows row0+4g+{0..3} then row0+16+4g+{0..3}, g = lane/16
// (this row set keeps the two reads of a half-wave on distinct LDS banks).
__device__ __forceinline__ FragBF trfrag(const __bf16 *tile, int ld, int row0, int col0, int li, int lg) {
  FragBF f;
  f.v = __builtin_shufflevector(tr4(tile, ld, row0 + 4 * lg, col0, li),
                                tr4(tile, ld, row0 + 16 + 4 * lg, col0, li), 0, 1, 2, 3, 4, 5, 6, 7);
  return f;
}
__device__ __forceinline__ FragF32 trfrag(const float *tile, int ld, int row0, int col0, int li, int lg) {
  FragF32 f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f.v[k] = tile[(row0 + 4 * lg + k) * ld + col0 + li];
    f.v[4 + k] = tile[(row0 + 16 + 4 * lg + k) * ld + col0 + li];
  }
  return f;
}
__device__ __forceinline__ float elem(const FragBF &f, int e) { return (float)f.v[e]; }
__device__ __forceinline__ float elem(const FragF32 &f, int e) { return f.v[e]; }

// Row stride (elements) of a tile read with transposed reads: at least
// 16 bytes of padding and a byte stride that is an odd multiple of 32, so
// the 8 rows read by a half-wave fall on distinct LDS banks.
constexpr int tr_ld(int cols, int esize) {
  int ld = cols + 16 / esize;
  while ((ld * esize) % 64 != 32) ++ld;
  return ld;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (gfx9 data-parallel primitives).
__device__ __forceinline__ float wave_incl_scan(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x111, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x112, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x114, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x118, 0xf, 0xf, true));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xa, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xc, 0xf, false));
  return v;
}

// Workgroup barrier that orders LDS accesses only: the wave's own LDS reads
// and writes complete before it arrives (lgkmcnt(0)); its global loads and
// stores and its buffer loads into LDS may stay in flight (HIP's
// __syncthreads waits for those too where a copy into LDS is pending).  A
// wave whose copy into LDS the others read waits for it (vmcnt(0)) before
// the barrier.  The empty asm statements keep the compiler from moving memory
// accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F); // lgkmcnt(0); vmcnt, expcnt not waited on
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// Sum over aligned groups of NL lanes (4, 8 or 16) in registers, with DPP
// inside a 16-lane row (no LDS round trip): swap neighbours, swap pairs,
// mirror within each half row, mirror the row.  Every lane of a group ends
// with the same value (each step adds two values in either order).
template <int CTRL> __device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int NL> __device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(NL == 4 || NL == 8 || NL == 16, "groups of 4, 8 or 16 lanes");
  v = dpp_add<0xB1>(v); // quad_perm [1,0,3,2]
  v = dpp_add<0x4E>(v); // quad_perm [2,3,0,1]
  if constexpr (NL >= 8) v = dpp_add<0x141>(v); // row_half_mirror
  if constexpr (NL >= 16) v = dpp_add<0x140>(v); // row_mirror
  return v;
}

} // namespace
} // namespace ssd
