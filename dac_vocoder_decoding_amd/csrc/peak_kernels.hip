// peak_kernels.hip -- microbenchmarks of what the MI355X delivers, reported
// beside the published peaks: a matrix-core loop per operand dtype (the
// same 16x16 MFMA fragments the convolutions issue).  The HBM side uses the
// plain copy kernel of stream_kernels.hip.
#include "internal.h"
#include "gemm_common.h"

namespace voc {

// Each wave runs kChains independent accumulator chains of mfma_frag (four
// 16x16x4 fp32 MFMAs, or one 16x16x32 bf16 MFMA) so that the matrix pipe
// never waits on a result; operands stay in registers; the sums are
// written out so that nothing is dead code.  Measured on MI355X with four
// workgroups of four waves per CU: 16 chains reach 155.5 TFLOP/s fp32
// (99 % of the published peak) and 2.2 PFLOP/s bf16 (88 %); 8 chains hold
// the bf16 shape to 1.4 PFLOP/s (its results are not ready for the next
// dependent step), and 8 workgroups per CU with 8 chains the fp32 one to
// 137 TFLOP/s.
constexpr int kChains = 16;

template <int OP>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int64_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  uint4 a, b;
  if constexpr (OP == OP_F32) {
    const float x = 1e-3f * static_cast<float>(lane + 1), y = 1e-3f * static_cast<float>(64 - lane);
    a = make_uint4(__float_as_uint(x), __float_as_uint(y), __float_as_uint(x), __float_as_uint(y));
    b = make_uint4(__float_as_uint(y), __float_as_uint(x), __float_as_uint(y), __float_as_uint(x));
  } else {
    const uint32_t x = pack_bf16x2(1e-3f * static_cast<float>(lane + 1), 1e-3f);
    const uint32_t y = pack_bf16x2(1e-3f, 1e-3f * static_cast<float>(64 - lane));
    a = make_uint4(x, y, x, y);
    b = make_uint4(y, x, y, x);
  }
  f4 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) acc[k] = f4{0.f, 0.f, 0.f, 0.f};
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kChains; ++k) mfma_frag<OP>(a, b, acc[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

// The 32x32 forms (fp32 32x32x2, bf16 32x32x16): 16 accumulators per lane.
typedef float f16v __attribute__((ext_vector_type(16)));

template <int OP>
__global__ __launch_bounds__(256) void mfma32_loop_kernel(int64_t iters, float* out) {
  const int lane = threadIdx.x & 63;
  f16v acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  if constexpr (OP == OP_F32) {
    const float x = 1e-3f * static_cast<float>(lane + 1), y = 1e-3f * static_cast<float>(64 - lane);
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(x, y, acc[k], 0, 0, 0);
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x2f32(y, x, acc[k], 0, 0, 0);
      }
    }
  } else {
    const uint32_t x = pack_bf16x2(1e-3f * static_cast<float>(lane + 1), 1e-3f);
    const uint32_t y = pack_bf16x2(1e-3f, 1e-3f * static_cast<float>(64 - lane));
    const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(x, y, x, y));
    const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(y, x, y, x));
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

int mfma_loop_blocks() { return 256 * 4; }  // 4 workgroups of 4 waves per CU

double mfma32_loop_flops(int op, int64_t iters) {
  const double per_iter = op == OP_F32 ? 4.0 * 2 * 32 * 32 * 2 * 2 : 4.0 * 32 * 32 * 16 * 2;
  return static_cast<double>(mfma_loop_blocks()) * 4 * iters * per_iter;
}

hipError_t launch_mfma32_loop(int op, int64_t iters, float* out, hipStream_t s) {
  const dim3 grid(mfma_loop_blocks()), block(256);
  if (op == OP_F32)
    hipLaunchKernelGGL(mfma32_loop_kernel<OP_F32>, grid, block, 0, s, iters, out);
  else
    hipLaunchKernelGGL(mfma32_loop_kernel<OP_BF16>, grid, block, 0, s, iters, out);
  return hipGetLastError();
}

double mfma_loop_flops(int op, int64_t iters) {
  const double per_frag = op == OP_F32 ? 4.0 * 16 * 16 * 4 * 2 : 16.0 * 16 * 32 * 2;
  return static_cast<double>(mfma_loop_blocks()) * 4 * iters * kChains * per_frag;
}

hipError_t launch_mfma_loop(int op, int64_t iters, float* out, hipStream_t s) {
  const dim3 grid(mfma_loop_blocks()), block(256);
  if (op == OP_F32)
    hipLaunchKernelGGL(mfma_loop_kernel<OP_F32>, grid, block, 0, s, iters, out);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<OP_BF16>, grid, block, 0, s, iters, out);
  return hipGetLastError();
}

}  // namespace voc
