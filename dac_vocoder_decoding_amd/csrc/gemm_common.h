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

// nt (<= NT) matrix-core steps over LDS fragments: step t multiplies the WMB
// A fragments at a_at(t, mb) with the WNB B fragments at b_at(t, nb).  The
// fragments of step t+1 are read into a second register set before step t's
// MFMAs issue, so LDS latency overlaps matrix work instead of stalling it.
// Callers pass an nt that is a constant after unrolling.
// PIN keeps that order against the scheduler, which otherwise re-serialises
// the reads to save registers; it pays where the extra registers cost no
// occupancy that matters (the 7-tap GEMM), not in the fused unit or the
// 2-tap GEMM (measured per kernel).
template <int OP, int WMB, int WNB, int NT, bool PIN, typename FA, typename FB>
__device__ __forceinline__ void mma_steps(f4 (&acc)[WMB][WNB], int nt, FA a_at, FB b_at) {
  uint4 A[2][WMB], B[2][WNB];
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) A[0][mb] = *reinterpret_cast<const uint4*>(a_at(0, mb));
#pragma unroll
  for (int nb = 0; nb < WNB; ++nb) B[0][nb] = *reinterpret_cast<const uint4*>(b_at(0, nb));
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t >= nt) break;
    const int cur = t & 1;
    if (t + 1 < nt) {
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb)
        A[cur ^ 1][mb] = *reinterpret_cast<const uint4*>(a_at(t + 1, mb));
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
        B[cur ^ 1][nb] = *reinterpret_cast<const uint4*>(b_at(t + 1, nb));
    }
#pragma unroll
    for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb) mfma_frag<OP>(A[cur][mb], B[cur][nb], acc[mb][nb]);
  }
  if constexpr (PIN) {
    // Step 0's reads, then per step the next step's reads followed by this
    // step's MFMAs.
    constexpr int kMfmaPerFrag = OP == OP_F32 ? 4 : 1;
    __builtin_amdgcn_sched_group_barrier(0x100, WMB + WNB, 0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t >= nt) break;
      if (t + 1 < nt) __builtin_amdgcn_sched_group_barrier(0x100, WMB + WNB, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, WMB * WNB * kMfmaPerFrag, 0);
    }
  }
}

template <int TAPS> struct HaloMax { static constexpr int v = 0; };
template <> struct HaloMax<7> { static constexpr int v = 54; };  // 6 * dilation 9
template <> struct HaloMax<2> { static constexpr int v = 1; };
template <> struct HaloMax<3> { static constexpr int v = 2; };   // k=3, or a strided conv's 3 frame groups

// LDS tiles hold rows of one 64-byte channel chunk in blocks of 16 rows.
// Inside a block the four 16-byte units of a row are stored unit-major:
// (row, unit) lives at (row / 16) * 1024 + unit * 256 + (row % 16) * 16.
// An MFMA fragment read (16 consecutive rows from any first row x 4 units,
// lane = unit * 16 + row offset) and a wave's staging store (16 rows x 4
// units) then touch every 256-byte run of LDS once, which gfx950 serves at
// its full ds_read_b128 rate (~240 B/clk/CU measured); padded row pitches
// (80, 144 bytes) and plain 64-byte rows measured half that.
constexpr int kRowBytes = 64;  // LDS bytes per tile row (no padding)
__device__ __forceinline__ int lds_off(int row, int unit) {
  return ((row >> 4) << 10) + (unit << 8) + ((row & 15) << 4);
}

// ---------------------------------------------------------------- LDS DMA
// Tiles are copied global -> LDS by buffer loads with the LDS flag: lane l's
// 16 bytes land at LDS byte (M0 + 16 l), so one wave instruction fills one
// 1 KB block of 16 rows x 4 units in exactly the lds_off layout when lane l
// reads row (l % 16), unit (l / 16).  No registers hold the data in flight,
// which lets a kernel keep several chunks in flight.  A buffer resource
// bounds every read to [base, base + bytes): offsets at or past the end,
// including negative ones (they wrap to large unsigned values), read as
// zero, which is the convolution's zero padding.  The loads count in vmcnt;
// the compiler does not see them, so kernels wait with wait_vm<N>() and
// synchronise with lds_barrier().
typedef int i4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i4 buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xffffu));  // stride 0
  r.z = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));                 // num_records
  r.w = 0x00020000;                                                               // 32-bit data format
  return r;
}

// LDS byte offset of a generic pointer to LDS (its low 32 bits).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// One wave-wide copy: 16 bytes at byte offset voff of rsrc -> LDS lds + 16 * lane.
// M0 carries the LDS address; the compiler reserves M0, so its value is saved
// and restored around the copy.  Writing M0 needs one wait state before an
// LDS-DMA instruction reads it.
__device__ __forceinline__ void dma16(i4 rsrc, uint32_t voff, uint32_t lds) {
  // lds is uniform across the wave; readfirstlane keeps it in an SGPR even
  // where the compiler cannot prove that.
  lds = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(lds)));
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds)
      : "memory");
}

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wave's LDS reads have completed.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// 16-byte unit idx of a tile of 64-byte rows -> (row, column).  A wave's 64
// lanes cover 16 consecutive rows x 4 columns: a global load reads 16 whole
// rows, and the LDS store at lds_off(row, column) is one linear 1 KB block.
__device__ __forceinline__ int unit_row(int idx) { return ((idx >> 6) << 4) + (idx & 15); }
__device__ __forceinline__ int unit_col(int idx) { return (idx >> 4) & 3; }

}  // namespace voc
