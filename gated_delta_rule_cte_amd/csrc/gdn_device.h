// Device-side helpers shared by the libgdn kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float bf2f(__bf16 b) { return static_cast<float>(b); }
// round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ __bf16 f2bf(float f) { return static_cast<__bf16>(f); }

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__bf16>(__bf16 x) { return static_cast<float>(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return f2bf(x); }

// ---------------------------------------------------------------------------
// Raw buffer loads.  A load through a buffer descriptor whose offset lies at or
// beyond the descriptor's byte range returns zeros, so masked loads need no
// branch or select: invalid lanes pass kOOB.  Branch-free loads also let a
// software-pipelined loop keep prefetched values in their destination
// registers (a select on a loaded value would force a wait for the load).
// ---------------------------------------------------------------------------
constexpr int kBufferWord3 = 0x00020000;  // raw, untyped, stride 0 (gfx9 family)
constexpr uint32_t kOOB = 0x80000000u;    // beyond every range used here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(uint4 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((__vector_size__(16)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store8(uint2 v, __amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef unsigned int u32x2 __attribute__((__vector_size__(8)));
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// 8-element vectors: the per-lane operand slice of one 16x32 MFMA fragment,
// and the unit of global <-> LDS copies (16 B of bf16, 32 B of fp32).
// ---------------------------------------------------------------------------
template <typename T> struct Vec8;
template <> struct Vec8<__bf16> {
  uint4 u;
  __device__ __forceinline__ static Vec8 zero() { Vec8 v; v.u = make_uint4(0, 0, 0, 0); return v; }
  __device__ __forceinline__ static Vec8 load(const __bf16* p) { Vec8 v; v.u = *reinterpret_cast<const uint4*>(p); return v; }
  __device__ __forceinline__ void store(__bf16* p) const { *reinterpret_cast<uint4*>(p) = u; }
  __device__ __forceinline__ float get(int j) const {
    const uint32_t w = (&u.x)[j >> 1];
    return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  __device__ __forceinline__ bf16x8 frag() const { return __builtin_bit_cast(bf16x8, u); }
  // 16 bytes at byte offset `off` of buffer `r` (zeros when out of range)
  __device__ __forceinline__ static Vec8 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Vec8 v; v.u = buf_load16(r, off); return v;
  }
  // store to byte offset `off` of buffer `r` (dropped when out of range)
  __device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t off) const {
    buf_store16(u, r, off);
  }
};
template <> struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ static Vec8 zero() { Vec8 v; v.a = make_float4(0, 0, 0, 0); v.b = v.a; return v; }
  __device__ __forceinline__ static Vec8 load(const float* p) {
    Vec8 v; v.a = reinterpret_cast<const float4*>(p)[0]; v.b = reinterpret_cast<const float4*>(p)[1]; return v;
  }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<float4*>(p)[0] = a; reinterpret_cast<float4*>(p)[1] = b;
  }
  __device__ __forceinline__ float get(int j) const { return j < 4 ? (&a.x)[j] : (&b.x)[j - 4]; }
  // 32 bytes at byte offset `off` of buffer `r` (zeros when out of range)
  __device__ __forceinline__ static Vec8 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    Vec8 v;
    v.a = __builtin_bit_cast(float4, buf_load16(r, off));
    v.b = __builtin_bit_cast(float4, buf_load16(r, off + 16u));
    return v;
  }
  // store to byte offset `off` of buffer `r` (dropped when out of range)
  __device__ __forceinline__ void bstore(__amdgpu_buffer_rsrc_t r, uint32_t off) const {
    buf_store16(__builtin_bit_cast(uint4, a), r, off);
    buf_store16(__builtin_bit_cast(uint4, b), r, off + 16u);
  }
};

// ---------------------------------------------------------------------------
// 16x16 output, K = 32 per call.  Fragment convention (both operands): lane l
// supplies row/col (l % 16) and the 8 contraction indices 8*(l/16) .. +7.
// Accumulator: lane l holds D[4*(l/16) + i][l % 16], i = 0..3.
// bf16 uses v_mfma_f32_16x16x32_bf16; fp32 issues eight v_mfma_f32_16x16x4_f32,
// instruction s pairing contraction index 8*(l/16) + s of both operands.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
  __device__ __forceinline__ static f4 mma(const Vec8<__bf16>& a, const Vec8<__bf16>& b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.frag(), b.frag(), c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  __device__ __forceinline__ static f4 mma(const Vec8<float>& a, const Vec8<float>& b, f4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.x, b.a.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.y, b.a.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.z, b.a.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.w, b.a.w, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.x, b.b.x, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.y, b.b.y, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.z, b.b.z, c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.w, b.b.w, c, 0, 0, 0);
    return c;
  }
};

// ---------------------------------------------------------------------------
// Transposed LDS fragment read (gfx950 ds_read_b64_tr_b16).  Within each
// 16-lane group, lane i receives element (i % 4) of the 8-byte reads of lanes
// 4j + i / 4, j = 0..3.  So if lane L of the group reads row r + L / 4,
// columns c + 4 (L % 4) .. +3 of a row-major 16-bit matrix, lane i gets column
// c + i of rows r .. r + 3.  Two such reads give the 8 contraction elements of
// an MFMA fragment whose contraction index runs down the rows:
//   lane l -> M[r0 + 8 (l / 16) + j][c0 + l % 16], j = 0..7.
// Requires 8-byte aligned rows (pitch * 2 % 8 == 0) and c0 % 4 == 0.
// ---------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ Vec8<__bf16> lds_tr_frag(const __bf16* m, int pitch, int r0, int c0, int lane) {
  const int L = lane & 15, g = lane >> 4;
  const __bf16* p0 = m + (r0 + 8 * g + (L >> 2)) * pitch + c0 + 4 * (L & 3);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0));
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 4 * pitch));
  Vec8<__bf16> v;
  v.u = make_uint4((uint16_t)a[0] | (uint32_t)(uint16_t)a[1] << 16, (uint16_t)a[2] | (uint32_t)(uint16_t)a[3] << 16,
                   (uint16_t)b[0] | (uint32_t)(uint16_t)b[1] << 16, (uint16_t)b[2] | (uint32_t)(uint16_t)b[3] << 16);
  return v;
}
// One transposed read on its own: lane l of group g = l / 16 reads row
// row0 + l % 16 / 4 (row0 may depend on g), columns c0 + 4 (l % 4) .. +3, and
// receives M[row0 + j][c0 + l % 16], j = 0..3, as 4 packed bf16.
__device__ __forceinline__ uint2 lds_tr4(const __bf16* m, int pitch, int row0, int c0, int lane) {
  const int L = lane & 15;
  const i16x4 a =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(m + (row0 + (L >> 2)) * pitch + c0 + 4 * (L & 3)));
  return make_uint2((uint16_t)a[0] | (uint32_t)(uint16_t)a[1] << 16, (uint16_t)a[2] | (uint32_t)(uint16_t)a[3] << 16);
}
// element j of 4 packed bf16, as float
__device__ __forceinline__ float bf4_get(uint2 v, int j) {
  const uint32_t w = j < 2 ? v.x : v.y;
  return __uint_as_float((j & 1) ? (w & 0xFFFF0000u) : (w << 16));
}

// fp32 has no transposed read: gather the same fragment element by element
__device__ __forceinline__ Vec8<float> lds_tr_frag(const float* m, int pitch, int r0, int c0, int lane) {
  const int L = lane & 15, g = lane >> 4;
  const float* p = m + (r0 + 8 * g) * pitch + c0 + L;
  Vec8<float> v;
  v.a = make_float4(p[0], p[pitch], p[2 * pitch], p[3 * pitch]);
  v.b = make_float4(p[4 * pitch], p[5 * pitch], p[6 * pitch], p[7 * pitch]);
  return v;
}

// ---------------------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (linear workgroup id i
// runs on XCD i % 8), and each XCD has its own L2.  This remap gives XCD x a
// contiguous range of logical ids (n / 8 of them, one more for the first
// n % 8 XCDs), so workgroups that read the same bytes (neighbouring logical
// ids) share one L2.  A bijection on [0, n) for every n.
// ---------------------------------------------------------------------------
constexpr int kXCDs = 8;
__device__ __forceinline__ int xcd_logical_id(int hw_id, int n) {
  const int q = n / kXCDs, r = n % kXCDs;
  const int x = hw_id % kXCDs, slot = hw_id / kXCDs;
  return x * q + (x < r ? x : r) + slot;
}

// ---------------------------------------------------------------------------
// wavefront reductions / scans (wave64)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}
// inclusive prefix sum over the 64 lanes (ds_bpermute based; any lane count)
__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xF, true));
}

// inclusive prefix sum over the 64 lanes with DPP row shifts and row
// broadcasts (no LDS round trip): Hillis-Steele inside each 16-lane row,
// then lane 15 of a row is added to the next row, lane 31 to rows 2 and 3.
// Must be called by the whole wave.
__device__ __forceinline__ float wave_inclusive_scan_dpp(float x) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  x += dpp_move<kRowShr | 1, 0xF>(x);
  x += dpp_move<kRowShr | 2, 0xF>(x);
  x += dpp_move<kRowShr | 4, 0xF>(x);
  x += dpp_move<kRowShr | 8, 0xF>(x);
  x += dpp_move<kRowBcast15, 0xA>(x);
  x += dpp_move<kRowBcast31, 0xC>(x);
  return x;
}

// (the hardware reciprocal, within 1 ulp, instead of a correctly rounded
// division: every use rounds the result or a product of it to bf16, or keeps
// it far inside the fp32 tolerance)
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
// log(1 + e^x); above 20 the correction e^-x is below fp32 resolution of x.
__device__ __forceinline__ float softplusf_(float x) { return x > 20.0f ? x : log1pf(__expf(x)); }

}  // namespace gdn
