// gfx950 building blocks: 16-bit element vectors (bf16 or fp16), MFMA, LDS
// transpose reads, XCD id.  Kernels are templates on the element type T
// (__bf16 or _Float16); inputs and outputs travel as raw 16-bit patterns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vattn {

template <class T>
using vec8 = T __attribute__((ext_vector_type(8)));
template <class T>
using vec2 = T __attribute__((ext_vector_type(2)));
typedef vec8<__bf16> bf16x8;
typedef vec8<_Float16> f16x8;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32) += A(32x16) * B(16x32), 16-bit in, fp32 accumulate.  Lane l holds
// A[l%32][8*(l/32) + j] and B[8*(l/32) + j][l%32] for j = 0..7, and
// D[8*(i/4) + 4*(l/32) + i%4][l%32] in acc[i] (verified on gfx950 for bf16;
// the fp16 instruction has the same shape and operand layout).
__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <class T>
__device__ inline vec8<T> as_v8(u32x4 v) { return __builtin_bit_cast(vec8<T>, v); }

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// source lane i names 4 consecutive bf16 at its address (a 16x4 matrix M,
// row i); result lane i' receives M[4j + i'/4][i'%4] for j = 0..3.  Pointing
// source lane i at row (r0 + i/4), column (c0 + 4*(i%4)) of a row-major tile
// therefore hands lane i' the 4 rows r0..r0+3 of column c0 + i'.
// `p` must point into LDS; the address-space cast keeps constant offsets
// foldable into the instruction's offset field.
__device__ inline s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

template <class T>
__device__ inline vec8<T> concat8(s16x4 lo, s16x4 hi) {
  s16x8 r = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(vec8<T>, r);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to a packed pair of T, round to nearest even (one
// v_cvt_pk_bf16_f32 or v_cvt_pk_f16_f32).
template <class T>
__device__ inline uint32_t pack2(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, vec2<T>));
}

template <class T>
__device__ inline uint16_t to_bits(float a) {
  const T x = (T)a;
  return __builtin_bit_cast(uint16_t, x);
}

template <class T>
__device__ inline vec8<T> pack8(float a0, float a1, float a2, float a3, float a4, float a5,
                                float a6, float a7) {
  u32x4 r;
  r[0] = pack2<T>(a0, a1);
  r[1] = pack2<T>(a2, a3);
  r[2] = pack2<T>(a4, a5);
  r[3] = pack2<T>(a6, a7);
  return as_v8<T>(r);
}

// XCD (accelerator complex die) executing this wave.
__device__ inline int xcc_id() {
  unsigned r;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(r));
  return (int)(r & 0xf);
}

// 2^x with the hardware's v_exp_f32 (no denormal rescaling: results below
// 2^-126 flush to zero, which is harmless for softmax weights).
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline u32x4 load16(const uint16_t* p) { return *(const u32x4*)p; }
__device__ inline void store16(uint16_t* p, u32x4 v) { *(u32x4*)p = v; }

}  // namespace vattn
