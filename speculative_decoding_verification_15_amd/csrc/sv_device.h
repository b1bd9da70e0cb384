// Device-side building blocks shared by the verification kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// D(32x32, fp32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l supplies A[l % 32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l % 32];
// accumulator register v of lane l holds D[8*(v/4) + 4*(l/32) + v%4][l % 32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the lane pair (l, l ^ 32).  v_permlane32_swap with the same
// register as both operands leaves, between its two results, lane l's own value
// and its partner's in every lane; combining the two results symmetrically
// gives the pair reduction without depending on which result is which.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// IEEE maximum (NaN-propagating) of the lane pair (l, l ^ 32) and of three
// values: unlike fmaxf they need no quieting of their inputs (which the compiler
// otherwise adds for values it cannot prove canonical, such as MFMA results and
// permlane outputs), and gfx950 has a three-input form.  For the softmax's
// maxima, whose inputs are finite or -inf, the result is the same.
__device__ __forceinline__ float fmaximum(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float halves_maximum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Eight OCP e4m3 codes (little-endian bytes of `lo`, then `hi`) -> eight bf16
// values, exactly: v_cvt_pk_f32_fp8 decodes two codes to fp32 and every e4m3
// value is representable in bf16, so the packing conversion does not round.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)b[0]; r[3] = (__bf16)b[1];
  r[4] = (__bf16)c[0]; r[5] = (__bf16)c[1]; r[6] = (__bf16)d[0]; r[7] = (__bf16)d[1];
  return r;
}

}  // namespace sv
