// Device-side helpers shared by the gfx950 kernels: vector types, MFMA wrappers,
// conversions, cross-lane exchanges and the runtime epilogue interpreter.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_args.hpp"

namespace fa {

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------------------
// MFMA wrappers (gfx950).  Operand layouts used throughout, for a wave of 64 lanes:
//   32x32xK: lane l holds A[row l%32][k-slots of half l/32], B[k-slots of half l/32][col l%32];
//            C[r][c] with c = l%32, r = 8*(i/4) + 4*(l/32) + i%4 for accumulator index i.
//   16x16xK: lane l holds A[row l%16][k-slots of group l/16], B[...][col l%16];
//            C[r][c] with c = l%16, r = 4*(l/16) + i.
// The k-slot assignment is the same function for A and B, so any consistent relabelling
// of the contraction index between the two operands gives the same product.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ i32x4 mfma16_i8(i32x4 a, i32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------------------
// Conversions
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
  return __uint_as_float(((unsigned)b) << 16);
}
// Two fp32 -> packed bf16x2, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  bf16x2 p;
  p[0] = (__bf16)lo;
  p[1] = (__bf16)hi;
  return __builtin_bit_cast(unsigned, p);
}
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
  f16x2 p;
  p[0] = (_Float16)lo;
  p[1] = (_Float16)hi;
  return __builtin_bit_cast(unsigned, p);
}
// Four signed bytes of w -> two packed bf16x2 (exact: |x| <= 128 fits bf16's 8-bit significand).
__device__ __forceinline__ u32x2 i8x4_to_bf16x4(unsigned w) {
  u32x2 r;
  r[0] = pack_bf16x2((float)(signed char)(w), (float)(signed char)(w >> 8));
  r[1] = pack_bf16x2((float)(signed char)(w >> 16), (float)(signed char)(w >> 24));
  return r;
}
// Four signed bytes of w -> two packed fp16x2, exact: byte b+128 is placed in the low
// mantissa bits of fp16 1024.0 (0x6400) and 1152.0 is subtracted.
__device__ __forceinline__ u32x2 i8x4_to_f16x4(unsigned w) {
  const unsigned u = w ^ 0x80808080u;
  f16x2 bias;
  bias[0] = (_Float16)-1152.0f;
  bias[1] = (_Float16)-1152.0f;
  // selector bytes: 4..7 pick from the first operand (0x64646464), 0..3 from u
  f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u)) + bias;
  f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x05030402u)) + bias;
  u32x2 r;
  r[0] = __builtin_bit_cast(unsigned, lo);
  r[1] = __builtin_bit_cast(unsigned, hi);
  return r;
}

// ---------------------------------------------------------------------------------------
// Cross-lane exchanges
// ---------------------------------------------------------------------------------------
// Reductions across lane pairs (l, l ^ 32) and (l, l ^ 16), on the VALU: v_permlane32_swap /
// v_permlane16_swap with both operands x leave x's partner value in one of the two results and
// x itself in the other, so a symmetric op of the two results is the pair reduction on every
// lane (no LDS round trip as with ds_bpermute).
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One IEEE fp32 multiply or add rounded on its own: kept out of the FMA contraction that the
// compiler otherwise applies across statements (a product feeding a sum).
__device__ __forceinline__ float mul_rn(float x, float y) {
#pragma clang fp contract(off)
  return x * y;
}
__device__ __forceinline__ float add_rn(float x, float y) {
#pragma clang fp contract(off)
  return x + y;
}

// ---------------------------------------------------------------------------------------
// Epilogue: ops applied in list order in fp32, each a separately rounded IEEE operation
// (no contraction into FMA), so the fused result equals the same ops applied on the host.
// Mul and Add take a scalar, Bias adds a per-channel vector (channel = head-dim index of the
// output element), ReLU maps x to x > 0 ? x : +0.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float epilogue_op(float x, int kind, float c, const float* vec, int channel) {
  if (kind == kEpiMul) return mul_rn(x, c);
  if (kind == kEpiAdd) return add_rn(x, c);
  if (kind == kEpiBias) return add_rn(x, vec[channel]);
  return x > 0.f ? x : 0.f;
}

__device__ __forceinline__ float apply_epilogue(float x, const EpiArgs& e, int channel) {
  for (int i = 0; i < e.n; ++i) x = epilogue_op(x, e.kind[i], e.value[i], e.vec[i], channel);
  return x;
}

// The same ops over an array, op-major (one uniform branch per op); channel(j) is the head-dim
// index of x[j].
template <int N, class Channel>
__device__ __forceinline__ void apply_epilogue_all(float (&x)[N], const EpiArgs& e, Channel channel) {
  for (int i = 0; i < e.n; ++i) {
    const int kind = e.kind[i];
    const float cv = e.value[i];
    if (kind == kEpiMul) {
#pragma unroll
      for (int j = 0; j < N; ++j) x[j] = mul_rn(x[j], cv);
    } else if (kind == kEpiAdd) {
#pragma unroll
      for (int j = 0; j < N; ++j) x[j] = add_rn(x[j], cv);
    } else if (kind == kEpiBias) {
      const float* vec = e.vec[i];
#pragma unroll
      for (int j = 0; j < N; ++j) x[j] = add_rn(x[j], vec[channel(j)]);
    } else {
#pragma unroll
      for (int j = 0; j < N; ++j) x[j] = x[j] > 0.f ? x[j] : 0.f;
    }
  }
}

// Score-scope ops over a tile's raw scores x[j] = q.k, before the mask and the softmax scale;
// key(j) is the key position of x[j], which the caller clamps into [0, s_k) so that a bias read
// stays inside its vector (scores of keys past the end are masked right after).
template <int N, class Key>
__device__ __forceinline__ void apply_score_ops(float (&x)[N], const EpiArgs& e, Key key) {
  apply_epilogue_all(x, e, key);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// Lanes of one wave exchanging data through a wave-private LDS slot: the hardware performs a
// wave's LDS accesses in order, so the compiler only has to keep them in program order, which it
// would not otherwise do where it can prove that one lane's own accesses do not overlap (no
// memory access moves across this).
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

}  // namespace fa
