// device_math.h -- elementwise device helpers of libvocoder: the Snake
// activation and float -> bfloat16 rounding.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace voc {

typedef float f4 __attribute__((ext_vector_type(4)));

// Snake / SnakeBeta: x + sin^2(alpha x) * invden, with invden = 1/(alpha+1e-9)
// (Snake, minimaxmusic.cpp ARCHITECTURE "Flow VAE") or 1/(beta+1e-9)
// (SnakeBeta, qwentts.cpp ARCHITECTURE glossary), precomputed at load.
//
// sin^2 has period pi, so z = alpha x is reduced to r = z - k pi with
// k = rint(z / pi) and |r| <= pi/2.  pi is split into PI_HI = float(pi) and
// PI_LO = pi - PI_HI (Cody & Waite, "Software Manual for the Elementary
// Functions", 1980); the k*PI_HI step is a fused multiply-add, so it is exact
// up to one rounding for every |k| this network reaches.  sin(r) is the
// Taylor series through r^13, whose truncation error on |r| <= pi/2 is below
// (pi/2)^15 / 15! < 7e-10.
__device__ __forceinline__ float snake_f32(float x, float alpha, float invden) {
  const float z = alpha * x;
  const float k = rintf(z * 0.318309886183790672f);
  float r = fmaf(-k, 3.14159274101257324f, z);
  r = fmaf(-k, -8.74227800037248e-08f, r);
  const float r2 = r * r;
  float p = 1.60590438368216146e-10f;            //  1/13!
  p = fmaf(p, r2, -2.50521083854417188e-08f);    // -1/11!
  p = fmaf(p, r2, 2.75573192239858907e-06f);     //  1/9!
  p = fmaf(p, r2, -1.98412698412698413e-04f);    // -1/7!
  p = fmaf(p, r2, 8.33333333333333333e-03f);     //  1/5!
  p = fmaf(p, r2, -1.66666666666666667e-01f);    // -1/3!
  p = fmaf(p, r2, 1.0f);
  const float s = r * p;
  return fmaf(s * s, invden, x);
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

template <>
__device__ __forceinline__ void store_op4<1>(void* base, int64_t idx, f4 v) {
  uint2 p;
  p.x = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
  p.y = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
  *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + idx) = p;
}

}  // namespace voc
