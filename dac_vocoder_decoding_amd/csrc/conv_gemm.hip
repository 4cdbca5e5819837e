// conv_gemm.hip -- implicit-GEMM convolutions on the gfx950 matrix cores.
//
// One kernel template serves every convolution of the decoder:
//   * Conv1d k=7 at dilation d (conv_in, residual conv1): 7 taps at frame
//     offsets j*d - 3d;
//   * Conv1d k=1 (residual conv2): 1 tap;
//   * ConvTranspose1d k=2s stride s as a polyphase GEMM: output phase r of
//     input frame q is x[q] w[:, :, r] + x[q-1] w[:, :, s+r], i.e. 2 taps at
//     offsets 0 and -1 with M = s*Cout rows m = r*Cout + o.  The transposed
//     conv is a scatter of kernel copies (the col2im_1d overlap-add of the
//     qwentts.cpp ARCHITECTURE page, "Custom GGML ops"); grouping the
//     scattered outputs by phase turns it into a dense GEMM with no column
//     matrix and no zero-stuffing.
//
// GEMM view: D[m][n] = sum_{tap, i} W[tap][m][i] * X[n + off(tap)][i],
// m = output feature, n = output position, reduction over input channels i
// (and taps).  The matrix-core "A" operand is the packed weight tile, "B" is
// the activation tile.  Per 64-byte channel chunk the workgroup stages
//   X rows [n0 + min_off, n0 + BN + max_off)  (the dilation halo included)
//   W      [TAPS][BM] rows
// into LDS once and every tap reads its shifted window of the same X tile.
// Loads for chunk c+1 are issued into registers before the matrix work of
// chunk c.  The epilogue adds the bias and optionally the residual, stores
// the fp32 result and/or the next layer's Snake of it in the operand dtype,
// so every Snake is evaluated once per element.
//
// Matrix-core instructions (16x16 output blocks, wave64):
//   fp32: v_mfma_f32_16x16x4_f32; bf16: v_mfma_f32_16x16x32_bf16.
// Lane l of a wave supplies row/column (l % 16) and the 16-byte slice
// (l / 16) of the 64-byte chunk; for fp32 the four floats of that slice feed
// four successive 16x16x4 steps (reduction index permuted consistently on
// both operands).  Accumulator register v of lane l holds D[4*(l/16)+v][l%16].
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

// TAG only separates kernel names per layer kind (conv_in vs residual k7)
// so that profilers report them apart; it does not change the code.
template <int OP, int TAPS, int WMB, int WNB, int WAVES_M, int WAVES_N, int TAG>
__global__ __launch_bounds__(256) void conv_gemm_kernel(const ConvArgs a) {
  constexpr int CH = OpT<OP>::CH;
  constexpr int ES = OpT<OP>::ES;
  constexpr int BM = WAVES_M * WMB * 16;
  constexpr int BN = WAVES_N * WNB * 16;
  constexpr int XROWS = BN + HaloMax<TAPS>::v;
  constexpr int WROWS = TAPS * BM;
  constexpr int XU = (XROWS * 4 + 255) / 256;
  constexpr int WU = (WROWS * 4 + 255) / 256;
  static_assert(WAVES_M * WAVES_N == 4, "four waves per workgroup");
  __shared__ __attribute__((aligned(16))) unsigned char Xs[XROWS * kLdsRow];
  __shared__ __attribute__((aligned(16))) unsigned char Ws[WROWS * kLdsRow];

  const int tid = threadIdx.x;
  const int total = a.n_tiles * a.m_tiles * a.rows;
  const int L = xcd_remap(blockIdx.x, total);
  const int n_tile = L % a.n_tiles;
  const int rest = L / a.n_tiles;
  const int m_tile = rest % a.m_tiles;
  const int row = rest / a.m_tiles;
  const int n0 = n_tile * BN;
  const int m0 = m_tile * BM;
  const int len = a.row_len[row];
  const int Lin = min(len * a.rate_in, a.T_in);
  const int Lout = min(len * a.rate_out, a.T_out);
  // The whole tile lies beyond this row's valid output: nothing to do.
  if (n0 * a.ups - a.crop >= Lout) return;

  const int xrows = BN + a.halo;
  const int tfirst = n0 + a.min_off;
  const int nchunks = a.Cin / CH;
  const unsigned char* xrow = static_cast<const unsigned char*>(a.x) +
                              static_cast<int64_t>(row) * a.Cin * a.T_in * ES;
  const int64_t xplane = static_cast<int64_t>(a.T_in) * kChunkBytes;
  const unsigned char* wbase = static_cast<const unsigned char*>(a.w);
  const int64_t wplane = static_cast<int64_t>(TAPS) * a.M * kChunkBytes;

  uint4 xr[XU], wr[WU];
  auto gload = [&](int c) {
    const unsigned char* xc = xrow + c * xplane;
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int idx = tid + u * 256;
      const int r = idx >> 2, col = idx & 3;
      const int t = tfirst + r;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (idx < xrows * 4 && t >= 0 && t < Lin)
        v = *reinterpret_cast<const uint4*>(xc + static_cast<int64_t>(t) * kChunkBytes + col * 16);
      xr[u] = v;
    }
    const unsigned char* wc = wbase + c * wplane;
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int idx = tid + u * 256;
      const int r = idx >> 2, col = idx & 3;
      const int j = r / BM, mm = r - j * BM;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (idx < WROWS * 4 && m0 + mm < a.M)
        v = *reinterpret_cast<const uint4*>(
            wc + (static_cast<int64_t>(j) * a.M + m0 + mm) * kChunkBytes + col * 16);
      wr[u] = v;
    }
  };
  auto lstore = [&]() {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int idx = tid + u * 256;
      if (idx < xrows * 4)
        *reinterpret_cast<uint4*>(Xs + (idx >> 2) * kLdsRow + (idx & 3) * 16) = xr[u];
    }
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int idx = tid + u * 256;
      if (idx < WROWS * 4)
        *reinterpret_cast<uint4*>(Ws + (idx >> 2) * kLdsRow + (idx & 3) * 16) = wr[u];
    }
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave % WAVES_M, wn = wave / WAVES_M;
  const int lr = lane & 15, lg = lane >> 4;

  f4 acc[WMB][WNB];
#pragma unroll
  for (int i = 0; i < WMB; ++i)
#pragma unroll
    for (int j = 0; j < WNB; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

  gload(0);
  for (int c = 0; c < nchunks; ++c) {
    lstore();
    __syncthreads();
    if (c + 1 < nchunks) gload(c + 1);
#pragma unroll
    for (int j = 0; j < TAPS; ++j) {
      const int xoff = a.off0 + j * a.offstep - a.min_off + wn * WNB * 16 + lr;
      uint4 A[WMB], B[WNB];
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb)
        A[mb] = *reinterpret_cast<const uint4*>(
            Ws + (j * BM + wm * WMB * 16 + mb * 16 + lr) * kLdsRow + lg * 16);
#pragma unroll
      for (int nb = 0; nb < WNB; ++nb)
        B[nb] = *reinterpret_cast<const uint4*>(Xs + (xoff + nb * 16) * kLdsRow + lg * 16);
#pragma unroll
      for (int mb = 0; mb < WMB; ++mb)
#pragma unroll
        for (int nb = 0; nb < WNB; ++nb) mfma_frag<OP>(A[mb], B[nb], acc[mb][nb]);
    }
    __syncthreads();
  }

  // Epilogue.
#pragma unroll
  for (int mb = 0; mb < WMB; ++mb) {
    const int m = m0 + wm * WMB * 16 + mb * 16 + lg * 4;
    if (m >= a.M) continue;
    const int ph = m / a.Cout;
    const int o = m - ph * a.Cout;
    const f4 bias = *reinterpret_cast<const f4*>(a.bias + o);
    f4 sal = f4{0.f, 0.f, 0.f, 0.f}, sinv = f4{0.f, 0.f, 0.f, 0.f};
    if (a.s_out) {
      sal = *reinterpret_cast<const f4*>(a.s_alpha + o);
      sinv = *reinterpret_cast<const f4*>(a.s_invden + o);
    }
    const int64_t hbase = (static_cast<int64_t>(row) * a.Cout + (o & ~15)) * a.T_out + (o & 15);
    const int64_t sbase = (static_cast<int64_t>(row) * a.Cout + (o / CH) * CH) * a.T_out + (o % CH);
#pragma unroll
    for (int nb = 0; nb < WNB; ++nb) {
      const int n = n0 + wn * WNB * 16 + nb * 16 + lr;
      if (n >= a.N) continue;
      const int tau = n * a.ups + ph - a.crop;
      if (tau < 0 || tau >= Lout) continue;
      f4 v = acc[mb][nb] + bias;
      const int64_t hidx = hbase + static_cast<int64_t>(tau) * kHChunk;
      if (a.res) v += *reinterpret_cast<const f4*>(a.res + hidx);
      if (a.h_out) *reinterpret_cast<f4*>(a.h_out + hidx) = v;
      if (a.s_out) {
        f4 sv;
        sv[0] = snake_f32(v[0], sal[0], sinv[0]);
        sv[1] = snake_f32(v[1], sal[1], sinv[1]);
        sv[2] = snake_f32(v[2], sal[2], sinv[2]);
        sv[3] = snake_f32(v[3], sal[3], sinv[3]);
        store_op4<OP>(a.s_out, sbase + static_cast<int64_t>(tau) * CH, sv);
      }
    }
  }
}

int conv_variant_bm(int v) { return v == CV_128x128 ? 128 : 64; }
int conv_variant_bn(int v) { return v == CV_64x256 ? 256 : 128; }
bool conv_variant_ok(int v, int taps) {
  // A 7-tap weight tile of 128 rows would not fit 64 KB of LDS.
  return !(taps == 7 && v == CV_128x128);
}

template <int OP, int TAPS, int TAG>
static hipError_t launch_taps(int variant, const ConvArgs& a, hipStream_t s) {
  const int total = a.n_tiles * a.m_tiles * a.rows;
  const dim3 grid(total), block(256);
  switch (variant) {
    case CV_64x256:
      hipLaunchKernelGGL((conv_gemm_kernel<OP, TAPS, 4, 4, 1, 4, TAG>), grid, block, 0, s, a);
      break;
    case CV_64x128:
      hipLaunchKernelGGL((conv_gemm_kernel<OP, TAPS, 4, 2, 1, 4, TAG>), grid, block, 0, s, a);
      break;
    case CV_128x128:
      if constexpr (TAPS != 7) {
        hipLaunchKernelGGL((conv_gemm_kernel<OP, TAPS, 4, 4, 2, 2, TAG>), grid, block, 0, s, a);
        break;
      }
      return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int OP>
static hipError_t launch_op(int taps, int variant, bool conv_in, const ConvArgs& a, hipStream_t s) {
  switch (taps) {
    case 7:
      return conv_in ? launch_taps<OP, 7, 1>(variant, a, s) : launch_taps<OP, 7, 0>(variant, a, s);
    case 2: return launch_taps<OP, 2, 0>(variant, a, s);
    case 1: return launch_taps<OP, 1, 0>(variant, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_conv(int op, int taps, int variant, bool conv_in, const ConvArgs& a,
                       hipStream_t s) {
  return op == OP_F32 ? launch_op<OP_F32>(taps, variant, conv_in, a, s)
                      : launch_op<OP_BF16>(taps, variant, conv_in, a, s);
}

}  // namespace voc
