// Device-side helpers shared by the gfx950 kernels of libpagedkv.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Index of the calling wave in its workgroup, as a value the compiler knows
// to be wave-uniform (an SGPR): loops bounded by it are then plain scalar
// loops instead of exec-masked divergent ones, whose merged exits make the
// compiler wait on loads still in flight.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// A value every lane of the wave holds identically (read from LDS or global
// memory at a uniform address), moved to an SGPR for the same reason.
__device__ __forceinline__ int32_t uniform(int32_t v) {
  return __builtin_amdgcn_readfirstlane(v);
}

// v_mfma_f32_16x16x32_bf16.  Lane l = 16*q + r supplies A[row r][k 8q..8q+7]
// and B[k 8q..8q+7][col r]; it receives C[rows 4q..4q+3][col r].
__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16.  Lane l = 32*h + r supplies A[row r][k 8h..8h+7]
// and B[k 8h..8h+7][col r]; element i of its result is
// C[row 8*(i/4) + 4*h + i%4][col r].
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16.  Within each group of 16 lanes, lane i receives, for
// e = 0..3, 16-bit element (i % 4) of the 8-byte chunk addressed by lane
// 4*e + i/4 of its group.  Addressing lane 4*e + m at row (base + e),
// column (c0 + 4*m) of a row-major 16-bit tile gives lane i the column
// (c0 + i) of rows base..base+3 -- a transposed 4x16 read.
__device__ __forceinline__ s16x4_t lds_read_tr16(const void* lds_ptr) {
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds_ptr));
}

__device__ __forceinline__ bf16x8_t cat_tr(s16x4_t lo, s16x4_t hi) {
  typedef short s16x8_t __attribute__((ext_vector_type(8)));
  s16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Eight OCP e4m3fn codes -> eight bf16 values (exact: every e4m3fn value is a
// bf16 value).  gfx950's v_cvt_scalef32_pk_bf16_fp8 decodes two OCP codes
// (the low or the high half of the word) straight to bf16; a scale of 1
// leaves the exponent as it is.
__device__ __forceinline__ bf16x8_t fp8x8_to_bf16(u32x2_t w) {
  const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  const bf16x8_t r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// (x of this lane, x of lane ^ 32), in some order, without an LDS round trip:
// v_permlane32_swap issued directly (this compiler folds the two results of
// __builtin_amdgcn_permlane32_swap(x, x, ...) into one); the nop covers a
// VALU write of the inputs right before it.
__device__ __forceinline__ void xor32_pair(float x, float& a, float& b) {
  a = x;
  b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float xor32_max(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float xor32_sum(float x) {
  float a, b;
  xor32_pair(x, a, b);
  return a + b;
}

// Compiler-only barrier: keeps LDS stores and loads of one wave in program
// order (the LDS itself processes one wave's requests in order).
__device__ __forceinline__ void order_lds() { asm volatile("" ::: "memory"); }

}  // namespace pkv
