// device_math.h -- elementwise device helpers of libvocoder: the Snake
// activation and float -> bfloat16 rounding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace voc {

typedef float f4 __attribute__((ext_vector_type(4)));

// Snake / SnakeBeta: x + sin^2(alpha x) / den with den = alpha + 1e-9
// (Snake, minimaxmusic.cpp ARCHITECTURE "Flow VAE") or beta + 1e-9
// (SnakeBeta, qwentts.cpp ARCHITECTURE glossary).
//
// With sin^2(t) = (1 - cos 2t) / 2 and the hardware cosine, whose argument is
// in revolutions (v_cos_f32 computes cos(2 pi r)):
//   cos(2 alpha x) = cos(2 pi r),  r = frac(x alpha / pi)   (v_fract_f32),
//   Snake(x) = x + h (1 - cos(2 pi r)),  h = 1 / (2 den).
// The per-channel parameters scale = alpha / pi and h are computed in fp64 at
// load.  Reducing r to [0, 1) keeps the hardware cosine in its accurate
// range; the phase error is that of the product x * scale, the same order as
// the rounding of alpha * x itself.
__device__ __forceinline__ float snake_f32(float x, float scale, float h) {
  const float r = __builtin_amdgcn_fractf(x * scale);
  const float c = __builtin_amdgcn_cosf(r);
  return fmaf(-h, c, x + h);
}

// Round-to-nearest-even float -> bfloat16 bits (finite inputs): add 0x7FFF
// plus the lowest kept bit, keep the top 16 bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_round(float f) {
  return __uint_as_float(f32_to_bf16_bits(f) << 16);
}

// Store four consecutive channels of an operand tensor.
template <int OP>
__device__ __forceinline__ void store_op4(void* base, int64_t idx, f4 v);

template <>
__device__ __forceinline__ void store_op4<0>(void* base, int64_t idx, f4 v) {
  *reinterpret_cast<f4*>(static_cast<float*>(base) + idx) = v;
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t p = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, p);
}

template <>
__device__ __forceinline__ void store_op4<1>(void* base, int64_t idx, f4 v) {
  uint2 p;
  p.x = pack_bf16x2(v[0], v[1]);
  p.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = p;
}

// Two-term bf16 operands: x is carried as hi = bf16(x) and lo = bf16(x - hi)
// (the difference is exact in fp32), and both terms meet the same bf16
// weights; the pair holds x to about 2^-17 of its magnitude.  bf16_lo4 gives
// the low term's fp32 value before its own rounding.
__device__ __forceinline__ f4 bf16_lo4(f4 v) {
  f4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = v[e] - bf16_round(v[e]);
  return r;
}

// The residual stream h, in the same [row][C/16][T][16] element layout for
// both operand dtypes: fp32 elements for fp32 operands, fp16 elements for
// bf16 operands (16-bit activations, at fp16's 11-bit mantissa: rounding h
// to fp16 after every stage moves the decode by under 2 % of the bf16
// operands' own error, where bf16 storage would add 40 %).  Arithmetic on h
// stays fp32; stores round to nearest even.  idx counts elements.
typedef _Float16 h4v __attribute__((ext_vector_type(4)));

template <int OP>
__device__ __forceinline__ f4 load_h4(const void* base, int64_t idx) {
  if constexpr (OP == 0) {
    return *reinterpret_cast<const f4*>(static_cast<const float*>(base) + idx);
  } else {
    return __builtin_convertvector(*reinterpret_cast<const h4v*>(static_cast<const _Float16*>(base) + idx), f4);
  }
}

// A freshly produced residual value as the stream holds it: every consumer
// (the stored h, the next layer's Snake operand, the head's Snake) starts
// from the same rounded value, so that an operand computed in a producer's
// epilogue equals one computed from the stored h.
template <int OP>
__device__ __forceinline__ f4 round_h4(f4 v) {
  if constexpr (OP == 0)
    return v;
  else
    return __builtin_convertvector(__builtin_convertvector(v, h4v), f4);
}

// Four residual values as loaded, converted only where they are used: fp16
// quads held this way take two VGPRs instead of four while they wait in
// registers (prefetched residuals, staged X tiles).  load_h4 == to_f4(load).
template <int OP> struct HQuad { typedef f4 T; };
template <> struct HQuad<1> { typedef h4v T; };

template <int OP>
__device__ __forceinline__ typename HQuad<OP>::T load_h4_raw(const void* base, int64_t idx) {
  if constexpr (OP == 0)
    return *reinterpret_cast<const f4*>(static_cast<const float*>(base) + idx);
  else
    return *reinterpret_cast<const h4v*>(static_cast<const _Float16*>(base) + idx);
}

template <int OP>
__device__ __forceinline__ f4 h4_to_f4(typename HQuad<OP>::T v) {
  if constexpr (OP == 0)
    return v;
  else
    return __builtin_convertvector(v, f4);
}

template <int OP>
__device__ __forceinline__ void store_h4(void* base, int64_t idx, f4 v) {
  if constexpr (OP == 0) {
    *reinterpret_cast<f4*>(static_cast<float*>(base) + idx) = v;
  } else {
    *reinterpret_cast<h4v*>(static_cast<_Float16*>(base) + idx) = __builtin_convertvector(v, h4v);
  }
}

}  // namespace voc
