// Device helpers shared by the kernels: E4M3 conversion, E4M3 encoding,
// vector types and wave64 reductions for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int v8i32 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// Two E4M3 codes (bytes 0-1 of w, or bytes 2-3 when HI) to two packed bf16,
// each exactly code value x 2**(exponent of `scale`) (the gfx950 scaled
// conversion reads only the exponent field of its fp32 scale operand, which
// is the E8M0 scale of the MXFP8 format).  E4M3 values are all exact in bf16.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, float scale) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, scale, HI));
}

// Eight codes held in two dwords to an MFMA operand of eight bf16 (element i
// from byte i).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1, float scale) {
  u32x4 r;
  r[0] = e4m3x2_to_bf16x2<false>(w0, scale);
  r[1] = e4m3x2_to_bf16x2<true>(w0, scale);
  r[2] = e4m3x2_to_bf16x2<false>(w1, scale);
  r[3] = e4m3x2_to_bf16x2<true>(w1, scale);
  return __builtin_bit_cast(bf16x8, r);
}

// Eight E4M3 codes (element i from byte i of w0:w1) times an fp32 scale:
// v[i] = fp32(code_i * s), one rounding of the exact product (the code's
// fp32 value is exact).
__device__ __forceinline__ void scaled_e4m3x8(uint32_t w0, uint32_t w1, float s, float (&v)[8]) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
  v[0] = a[0] * s;
  v[1] = a[1] * s;
  v[2] = b[0] * s;
  v[3] = b[1] * s;
  v[4] = c[0] * s;
  v[5] = c[1] * s;
  v[6] = d[0] * s;
  v[7] = d[1] * s;
}

// fp32 operand carrying an E8M0 scale byte in its exponent field.
__device__ __forceinline__ float e8m0_as_scale_operand(uint32_t u) {
  return __builtin_bit_cast(float, u << 23);
}

// Exact fp32 value of one E4M3 code (byte 0 of w).
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
}

// Nearest E4M3 code of an fp32 value, ties to even, saturating at +-448 (the
// hardware conversion rounds to nearest even and turns magnitudes >= 464
// into NaN, so the value is clamped first; the clamp keeps the sign of zero).
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  y = fminf(fmaxf(y, -448.0f), 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xffu;
}

// Two fp32 to two packed bf16, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float a) {
  return (uint16_t)(pack_bf16x2(a, 0.0f) & 0xffffu);
}

__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Reductions over the lane pairs (l, l ^ 16) and (l, l ^ 32) with the
// gfx950 row-swap moves (v_permlane16_swap / v_permlane32_swap): each lane
// gets both values of its pair from VALU moves, with no LDS round trip.
// Max and sum of two values do not depend on their order, so the results
// equal those of a xor shuffle.
__device__ __forceinline__ float pair_max16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_max32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair_sum16(float v) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float pair_sum32(float v) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// Inclusive prefix sum over the 64 lanes with DPP moves: shifts by 1, 2, 4, 8
// within each 16-lane row, then each row adds the totals of the rows before
// it (broadcasts of lanes 15 and 31).  Lanes a move has no source for add 0.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return x;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <typename T>
__device__ __forceinline__ T ld_global(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

// Streaming load (non-temporal hint): for data read once, such as KV codes.
// Measured on MI355X, a plain read kernel gains ~10% with the hint.
template <typename T>
__device__ __forceinline__ T ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
}

// 16-byte loads and stores for data exchanged between workgroups of one
// launch: they carry the sc1 cache policy, as agent-scope atomic accesses do
// on this part, so they are coherent across the per-XCD L2 caches.  The
// buffer resource covers `bytes` bytes from `base` (accesses beyond it read
// zero and write nothing).
constexpr int kCachePolicySC1 = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ f32x4 ld_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicySC1));
}

__device__ __forceinline__ void st_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kCachePolicySC1);
}

}  // namespace fp8pa
