// Device helpers shared by the CSA kernels (gfx950, wave64).
//
// MFMA operand layouts used throughout (lane l, g = l / 16, r = l % 16):
//  * v_mfma_f32_16x16x128_f8f6f4 (FP8 E4M3 A and B, unit scales):
//      A[m = r][k = 32g .. 32g+31] (32 bytes per lane), B[k = 32g..][n = r],
//      C[m = 4g + i][n = r] for i = 0..3.
//  * v_mfma_f32_32x32x64_f8f6f4 (FP8 A and B, unit scales):
//      A[m = l % 32][k = 32 (l / 32) .. + 31], B[k = 32 (l / 32) ..][n = l % 32],
//      C[m = (i / 4) 8 + (l / 32) 4 + i % 4][n = l % 32] for i = 0..15.
//  * v_mfma_f32_16x16x32_fp8_fp8 and v_mfma_f32_16x16x32_bf16:
//      A[m = r][k = 8g .. 8g+7], B[k = 8g..][n = r], C as above.
//  Only the pairing matters for correctness: byte/element e of lane l's A
//  and B operands multiply each other.
//
// LDS transpose reads (ds_read_b64_tr_b8 / _tr_b16) work on groups of 16
// lanes; within a group, lane j receives
//   tr_b8 : byte  e (e = 0..7) = byte  (j % 8) of the 8-byte row addressed by
//           group lane 2e + (j >= 8)
//   tr_b16: half  e (e = 0..3) = half  (j % 4) of the 8-byte row addressed by
//           group lane (j / 4) + 4e
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

#define CSA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---- MFMA wrappers -------------------------------------------------------
__device__ __forceinline__ v4f mfma_f8_128(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v16f mfma_f8_32x32(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_f8_32(long a, long b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_bf16_32(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- workgroup barrier for LDS traffic only -----------------------------
// Waits for this wave's LDS accesses (lgkmcnt(0)) but leaves global loads
// and LDS DMAs in flight, unlike __syncthreads, which also drains vmcnt.
// The empty asm statements keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0); vmcnt, expcnt unchanged
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- cross-lane reductions over the four 16-lane groups ------------------
// v_permlane32_swap(a, b) returns (a, b) with the upper half's a swapped
// for the lower half's b: lanes 0..31 get (a, a[l + 32]), lanes 32..63 get
// (b[l - 32], b).  So swap(x, x) leaves lane l holding (x[l & 31],
// x[(l & 31) + 32]).  v_permlane16_swap does the same for rows of 16 within
// each half (partner lane l ^ 16).
__device__ __forceinline__ float sum_over_groups(float x) {
  int xi = __float_as_int(x);
  auto a = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  float y = __int_as_float(a[0]) + __int_as_float(a[1]);
  int yi = __float_as_int(y);
  auto b = __builtin_amdgcn_permlane16_swap(yi, yi, false, false);
  return __int_as_float(b[0]) + __int_as_float(b[1]);
}
__device__ __forceinline__ float max_over_groups(float x) {
  int xi = __float_as_int(x);
  auto a = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  float y = fmaxf(__int_as_float(a[0]), __int_as_float(a[1]));
  int yi = __float_as_int(y);
  auto b = __builtin_amdgcn_permlane16_swap(yi, yi, false, false);
  return fmaxf(__int_as_float(b[0]), __int_as_float(b[1]));
}

// ---- number formats ------------------------------------------------------
// Two floats -> two BF16 values (round to nearest even) packed low, high in
// a 32-bit word: one v_cvt_pk_bf16_f32 on gfx950.
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){lo, hi}, v2bf));
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Four floats -> four E4M3 bytes (RNE, OCP E4M3FN on gfx950) packed in an int.
__device__ __forceinline__ int pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}
// E4M3 byte `sel` (0..3) of `w` -> float (exact).
__device__ __forceinline__ float fp8_to_f32(int w, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8(w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8(w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8(w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8(w, 3);
  }
}

// Smallest power of two s with amax / s <= 448 (E4M3 max), for finite
// amax >= 2^-100; 1 otherwise.  Exact: built from amax's exponent bits.
__device__ __forceinline__ float e4m3_pow2_scale(float amax) {
  if (!(amax >= 7.8886091e-31f) || !(amax < 3.0e38f)) return 1.0f;
  uint32_t u = __float_as_uint(amax);
  int e = (int)((u >> 23) & 0xff) - 127;          // amax = 2^e * f, f in [1, 2)
  int k = ((u & 0x7fffffu) <= 0x600000u) ? e - 8 : e - 7;   // f <= 1.75 ?
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t float_order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse rotary embedding of the output's rope dims ("DSV4 Audit -- Decode
// Repetition + Precision / Tensor-Core Plan", A4: the attention output is
// rotated by RoPE(-pos) at the query position, which turns the absolute
// positions carried by the summed keys into relative ones).  Rope dims pair
// up as (2i, 2i + 1) with frequency theta^(-2i / d_rope); the returned
// (cos, sin) are those of the angle -pos * theta^(-2i / d_rope).  The angle is
// formed and reduced to [-pi, pi] in FP64, so that the FP32 sin/cos keep
// their accuracy at positions near 2^31.
__device__ __forceinline__ float2 inv_rope_cs(int pos, int pair, int d_rope, double log2_theta) {
  const double f = exp2(-(double)(2 * pair) / (double)d_rope * log2_theta);
  double a = (double)pos * f;
  a -= 6.283185307179586 * rint(a * 0.15915494309189535);
  float s, c;
  sincosf(-(float)a, &s, &c);
  return make_float2(c, s);
}
// (x, y) rotated by the angle whose cosine and sine are cs.
__device__ __forceinline__ float2 rotate2(float x, float y, float2 cs) {
  return make_float2(x * cs.x - y * cs.y, x * cs.y + y * cs.x);
}

__device__ __forceinline__ v4i ld16(const void* p) { return *reinterpret_cast<const v4i*>(p); }

}  // namespace csa
