// gemm_common.h -- device building blocks shared by the matrix-core kernels
// of libvocoder: operand traits, the XCD-aware workgroup remap, one
// 16x16 output block's matrix-core step per 64-byte fragment, and the
// LDS tile geometry.
#pragma once
#include "internal.h"
#include "device_math.h"

namespace voc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <int OP> struct OpT;
template <> struct OpT<OP_F32> { static constexpr int CH = 16, ES = 4; };
template <> struct OpT<OP_BF16> { static constexpr int CH = 32, ES = 2; };

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup id % 8).
// Give each XCD a contiguous range of logical tiles so that tiles sharing a
// weight slice (same m-tile) and neighbouring activation rows stay in one
// XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = bid & 7, local = bid >> 3;
  return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

template <int OP>
__device__ __forceinline__ void mfma_frag(const uint4& a, const uint4& b, f4& acc);

template <>
__device__ __forceinline__ void mfma_frag<OP_F32>(const uint4& a, const uint4& b, f4& acc) {
  const f4 av = __builtin_bit_cast(f4, a);
  const f4 bv = __builtin_bit_cast(f4, b);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bv[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], bv[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], bv[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[3], bv[3], acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_frag<OP_BF16>(const uint4& a, const uint4& b, f4& acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

template <int TAPS> struct HaloMax { static constexpr int v = 0; };
template <> struct HaloMax<7> { static constexpr int v = 54; };  // 6 * dilation 9
template <> struct HaloMax<2> { static constexpr int v = 1; };

constexpr int kLdsRow = 80;  // 64-byte chunk row + 16 bytes: conflict-free ds_read_b128

// 16-byte unit idx of a tile of 64-byte rows -> (row, column).  A wave's 64
// lanes cover 16 consecutive rows x 4 columns, so a global load reads 16
// whole rows and an LDS store, like the fragment reads, touches 16
// different rows per column: no bank conflicts with the 80-byte row pitch.
__device__ __forceinline__ int unit_row(int idx) { return ((idx >> 6) << 4) + (idx & 15); }
__device__ __forceinline__ int unit_col(int idx) { return (idx >> 4) & 3; }

}  // namespace voc
