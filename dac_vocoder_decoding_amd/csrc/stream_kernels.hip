// stream_kernels.hip -- the bandwidth-bound kernels of libvocoder:
//   fold_kernel          weight-norm fold (fp64 norms), cast and repack (load
//                        time), including the encoder's phase-packed strided conv
//   import_kernel        [row][C][T] fp32 -> chunked operand / residual layouts,
//                        with the row gather of tiles, windows and streams
//   audio_import_kernel  mono audio -> a one-chunk operand (the encoder's input)
//   layer_state_kernel   a stream layer's carried context in and out
//   export_kernel        chunked fp32 -> [row][C][T] (stage runner, encoder output)
//   af_snake_kernel      alias-free Snake: 2x upsample, Snake, 2x downsample
//   snake_kernel         plain elementwise Snake (the split ablation)
//   col2im_kernel        overlap-add of a GEMM + col2im ConvTranspose1d (ablation)
//   head_kernel          Snake -> Conv1d k=7 to one or two channels -> bias ->
//                        tanh, with the tile / window crop folded into the store
//   tanh_kernel          standalone in-place tanh (the split tanh ablation)
//   copy_kernel          plain 16-byte vector copy (byte-counter calibration)
#include "internal.h"
#include "device_math.h"

#include <algorithm>

namespace voc {

// ---------------------------------------------------------------- fold
// Weight norm (minimaxmusic.cpp ARCHITECTURE, "Models"): w = g v / ||v||,
// the norm over each slice along axis 0 of the stored tensor; with g NULL
// (dec_in_proj, which has no weight norm) w = v.  One workgroup
// per slice; the sum of squares is accumulated in fp64.  The folded value is
// rounded fp64 -> fp32 (the F32 inference weights), then for bf16 operands
// to bf16 (round to nearest even), and written at its packed position.
__global__ __launch_bounds__(256) void fold_kernel(const FoldArgs a) {
  __shared__ double red[256];
  const int64_t i = blockIdx.x;
  const float* v = a.v + i * a.rest;
  double ss = 0.0;
  for (int64_t e = threadIdx.x; e < a.rest; e += 256) {
    const double x = v[e];
    ss += x * x;
  }
  red[threadIdx.x] = ss;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double n = sqrt(red[0]);
  if (threadIdx.x == 0) a.norms[i] = n;
  const bool plain = a.g == nullptr;  // a weight without weight norm: used as stored
  const double g = plain ? 1.0 : a.g[i];
  const int ch = a.op == OP_F32 ? 16 : 32;
  for (int64_t e = threadIdx.x; e < a.rest; e += 256) {
    const float wf = plain ? v[e] : static_cast<float>(g * static_cast<double>(v[e]) / n);
    int64_t idx;
    if (a.kind == PACK_CONV) {  // (Cout, Cin, K), slice = o
      const int ci = static_cast<int>(e / a.k), kk = static_cast<int>(e % a.k);
      idx = ((static_cast<int64_t>(ci / ch) * a.k + kk) * a.cout + i) * ch + ci % ch;
    } else if (a.kind == PACK_DOWN) {  // strided conv (Cout, Cin, 2s), slice = o
      // Kernel index j = q*s + p: phase p, tap q in {0, 1} of virtual chunk
      // (ci / ch) * s + p (the strided form in conv_gemm.hip).
      const int ci = static_cast<int>(e / a.k), j = static_cast<int>(e % a.k);
      const int q = j / a.stride, ph = j % a.stride;
      const int64_t vc = static_cast<int64_t>(ci / ch) * a.stride + ph;
      idx = ((vc * 2 + q) * a.cout + i) * ch + ci % ch;
    } else if (a.kind == PACK_CONVT) {  // (Cin, Cout, 2s), slice = ci
      const int o = static_cast<int>(e / (2 * a.stride));
      const int kk = static_cast<int>(e % (2 * a.stride));
      const int t = kk / a.stride, r = kk % a.stride;
      const int64_t M = static_cast<int64_t>(a.stride) * a.cout;
      idx = ((static_cast<int64_t>(i / ch) * 2 + t) * M + static_cast<int64_t>(r) * a.cout + o) * ch +
            i % ch;
    } else {  // PACK_HEAD (O, C, K), slice = o -> fp32 [O][K][C]
      const int ci = static_cast<int>(e / a.k), kk = static_cast<int>(e % a.k);
      static_cast<float*>(a.out)[(i * a.k + kk) * a.cin + ci] = a.round_bf16 ? bf16_round(wf) : wf;
      continue;
    }
    if (a.op == OP_F32)
      static_cast<float*>(a.out)[idx] = wf;
    else
      static_cast<uint16_t*>(a.out)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(wf));
  }
}

hipError_t launch_fold(const FoldArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fold_kernel, dim3(static_cast<unsigned>(a.d0)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// -------------------------------------------------------------- import
// Tile of 64 frames x 16 channels: coalesced reads along time, then writes
// of 4 consecutive channels per thread into the chunked layouts.
template <int OP>
__global__ __launch_bounds__(256) void import_kernel(const ImportArgs a) {
  constexpr int CH = OP == OP_F32 ? 16 : 32;
  __shared__ float tile[16][65];
  const int r = blockIdx.y;
  const int cblocks = a.C / 16;
  const int c0 = (blockIdx.x % cblocks) * 16;
  const int t0 = (blockIdx.x / cblocks) * 64;
  const int Tw = a.T_write > 0 ? a.T_write : a.T;  // frames written per row
  const int len = min(a.rows.len[r], Tw);
  const int sb = a.rows.src_b[r];
  const int64_t st = a.rows.start[r];
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = i * 4 + (tid >> 6), t = tid & 63;
    const int tt = t0 + t;
    float v = 0.f;
    if (tt < len) v = a.x[(static_cast<int64_t>(sb) * a.C + c0 + c) * a.T_src + st + tt];
    tile[c][t] = v;
  }
  __syncthreads();
  const int t = tid >> 2, c = (tid & 3) * 4;
  const int tt = t0 + t;
  if (tt >= Tw) return;
  f4 v;
  v[0] = tile[c][t];
  v[1] = tile[c + 1][t];
  v[2] = tile[c + 2][t];
  v[3] = tile[c + 3][t];
  const int cc = c0 + c;
  if (a.h_out) {
    if (a.s_out) v = round_h4<OP>(v);  // x is a residual value: the operand starts from the stored one
    const int64_t hidx = (static_cast<int64_t>(r) * a.C + (cc & ~15)) * a.T +
                         static_cast<int64_t>(tt) * kHChunk + (cc & 15);
    f4 hv = v;
    if (a.h_scale) {
#pragma unroll
      for (int e = 0; e < 4; ++e) hv[e] = snake_f32(v[e], a.h_scale[cc + e], a.h_h[cc + e]);
    }
    store_h4<OP>(a.h_out, hidx, hv);
  }
  if (a.s_out) {
    if (a.s_alpha) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = snake_f32(v[e], a.s_alpha[cc + e], a.s_invden[cc + e]);
    }
    const int64_t sidx = (static_cast<int64_t>(r) * a.C + (cc / CH) * CH) * a.T +
                         static_cast<int64_t>(tt) * CH + cc % CH;
    store_op4<OP>(a.s_out, sidx, v);
  }
}

hipError_t launch_import(const ImportArgs& a, hipStream_t s) {
  const int Tw = a.T_write > 0 ? a.T_write : a.T;
  const dim3 grid(static_cast<unsigned>((a.C / 16) * ((Tw + 63) / 64)),
                  static_cast<unsigned>(a.nrows));
  if (a.op == OP_F32)
    hipLaunchKernelGGL(import_kernel<OP_F32>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(import_kernel<OP_BF16>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// -------------------------------------------------------- audio import
// Mono audio rows [src][T] -> an operand tensor of one 64-byte channel chunk
// per frame whose channel 0 is the sample and the others zero (the
// encoder's conv_in has one input channel; its packed weights are zero past
// channel 0).
template <int OP>
__global__ __launch_bounds__(256) void audio_import_kernel(const float* x, void* out, int64_t T, int rows) {
  const int64_t total = static_cast<int64_t>(rows) * T;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    uint4* row = reinterpret_cast<uint4*>(static_cast<unsigned char*>(out) + i * kChunkBytes);
    uint4 first = make_uint4(0u, 0u, 0u, 0u);
    if constexpr (OP == OP_F32)
      first.x = __float_as_uint(x[i]);
    else
      first.x = pack_bf16x2(x[i], 0.f);
    row[0] = first;
    row[1] = row[2] = row[3] = make_uint4(0u, 0u, 0u, 0u);
  }
}

hipError_t launch_audio_import(int op, const float* x, void* out, int64_t T, int rows, hipStream_t s) {
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((rows * T + 255) / 256, 4096));
  if (op == OP_F32)
    hipLaunchKernelGGL(audio_import_kernel<OP_F32>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x,
                       out, T, rows);
  else
    hipLaunchKernelGGL(audio_import_kernel<OP_BF16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x,
                       out, T, rows);
  return hipGetLastError();
}

// -------------------------------------------------------------- export
template <int OP>
__global__ __launch_bounds__(256) void export_kernel(const void* h, float* y, int C, int T) {
  __shared__ float tile[16][65];
  const int r = blockIdx.y;
  const int cblocks = C / 16;
  const int c0 = (blockIdx.x % cblocks) * 16;
  const int t0 = (blockIdx.x / cblocks) * 64;
  const int tid = threadIdx.x;
  {
    const int t = tid >> 2, c = (tid & 3) * 4;
    const int tt = t0 + t;
    f4 v = f4{0.f, 0.f, 0.f, 0.f};
    if (tt < T)
      v = load_h4<OP>(h, (static_cast<int64_t>(r) * C + c0) * T + static_cast<int64_t>(tt) * kHChunk + c);
    tile[c][t] = v[0];
    tile[c + 1][t] = v[1];
    tile[c + 2][t] = v[2];
    tile[c + 3][t] = v[3];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = i * 4 + (tid >> 6), t = tid & 63;
    const int tt = t0 + t;
    if (tt < T) y[(static_cast<int64_t>(r) * C + c0 + c) * T + tt] = tile[c][t];
  }
}

hipError_t launch_export(int op, const void* h, float* y, int rows, int C, int T, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((C / 16) * ((T + 63) / 64)), static_cast<unsigned>(rows));
  if (op == OP_F32)
    hipLaunchKernelGGL(export_kernel<OP_F32>, grid, dim3(256), 0, s, h, y, C, T);
  else
    hipLaunchKernelGGL(export_kernel<OP_BF16>, grid, dim3(256), 0, s, h, y, C, T);
  return hipGetLastError();
}

// ---------------------------------------------------- stream layer state
// One layer's carried context in a stream (qwentts.cpp ARCHITECTURE,
// "Streaming decode (stateful path)": each causal conv keeps the last
// (K-1)*d rows of its input).  The layer's input buffer holds, per plane of
// frame rows (64-byte operand rows, or 16 residual-stream elements), the
// chunk in frames [0, Tr) and room for ctx frames before it.  The margin receives the saved context (old), and the new
// context (the last ctx frames of old followed by the chunk) is saved for the
// next chunk.  Margin writes (frames < 0) and chunk reads (frames >= 0) never
// overlap; old and new are separate buffers.
__global__ __launch_bounds__(256) void layer_state_kernel(const LayerStateArgs a) {
  const int U = a.row_bytes / 16;  // 16-byte units per frame row
  const int64_t rb = a.row_bytes;
  const int64_t total = a.planes * a.ctx * U;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < total;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t p = i / (a.ctx * U);
    const int k = static_cast<int>((i / U) % a.ctx), u = static_cast<int>(i % U);
    const uint4* old_row = reinterpret_cast<const uint4*>(a.old_state + (p * a.ctx + k) * rb) + u;
    unsigned char* plane = a.buf + p * a.plane_bytes;
    const uint4 o = *old_row;
    const int q = a.Tr + k;  // position in (old context, chunk)
    const uint4 nv = q < a.ctx ? *(reinterpret_cast<const uint4*>(a.old_state + (p * a.ctx + q) * rb) + u)
                               : *(reinterpret_cast<const uint4*>(plane + static_cast<int64_t>(q - a.ctx) * rb) + u);
    *(reinterpret_cast<uint4*>(plane + static_cast<int64_t>(k - a.ctx) * rb) + u) = o;
    *(reinterpret_cast<uint4*>(a.new_state + (p * a.ctx + k) * rb) + u) = nv;
  }
}

hipError_t launch_layer_state(const LayerStateArgs& a, hipStream_t s) {
  if (a.row_bytes <= 0 || a.row_bytes % 16) return hipErrorInvalidValue;
  const int64_t total = a.planes * a.ctx * (a.row_bytes / 16);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((total + 255) / 256, 2048));
  hipLaunchKernelGGL(layer_state_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- head
// Output head (minimaxmusic.cpp ARCHITECTURE, "Flow VAE": snake_out, conv_out
// k=7 with bias, tanh; two output channels for a decoder that writes stereo
// from one latent, as the H3 audio VAE of the TensorSharp minimax-h3 page
// does).  Its input holds Snake_out(h) in fp32 (applied by its producer), or
// (SNK, bf16 decoders) the fp16 residual stream h itself, to which the head
// applies Snake_out as it loads: half the bytes, and the Snake starts from
// the stored h as every other consumer's does.  The head is a pure stream:
//   lane l of a wave reads frame f = o0 - P + l (all C channels, 64-byte
//   chunk rows) and forms the seven per-tap projections of each output
//   channel, z_j[f] = sum_i w[j][i] x[f][i];
//   lane l (P <= l < P + 58) then owns output o = f and gathers
//   y[o] = tanh(bias + sum_j z_j[o + j - P]) from lanes l + j - P with
//   cross-lane shuffles.  P = 3 for the "same" conv, 6 for the causal one
//   (qwentts.cpp ARCHITECTURE, "Streaming decode": every module causal).
// Each wave emits 58 outputs per 64 frames read; no LDS tile, no barriers.
// Frames outside the row's valid range [-lb, len) read as zero (the conv's
// zero padding; Snake(0) = 0; lb > 0 only for a stream's carried context).  The tile crop of time-tiled decoding is folded
// into the store.
constexpr int kHeadOut = 58;  // outputs per wave

template <int NOUT, int SNK>
__global__ __launch_bounds__(256) void head_kernel(const HeadArgs a) {
  const int r = blockIdx.y;
  const int lo = a.rows.keep_lo[r], hi = a.rows.keep_hi[r];
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int o0 = lo + wave * kHeadOut;
  if (o0 >= hi) return;
  const int C = a.C;
  const int Lr = min(a.rows.len[r] * a.rate, a.T);
  const int P = a.pad;  // 3, or 6 for the causal head
  const int f = o0 - P + lane;
  const bool valid = f >= -a.lb && f < Lr;
  const int64_t hp = static_cast<int64_t>(r) * C * a.T + static_cast<int64_t>(f) * kHChunk;
  const int64_t plane = static_cast<int64_t>(a.T) * kHChunk;
  float z[NOUT][7];
#pragma unroll
  for (int oc = 0; oc < NOUT; ++oc)
#pragma unroll
    for (int j = 0; j < 7; ++j) z[oc][j] = 0.f;
  // Chunks are read four at a time (256 bytes per lane in flight): 3 %
  // faster than one at a time on the batched bf16 windows (4.7 against 4.55
  // TB/s).  Non-temporal loads were 1.7x slower: each lane reads a 64-byte
  // row as four 16-byte pieces, which then reach HBM unmerged.
  constexpr int U = 4;
  const int nk = C / 16;
  for (int k0 = 0; k0 < nk; k0 += U) {
    f4 x[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        x[u][q] = valid && k0 + u < nk ? load_h4<SNK>(a.h, hp + (k0 + u) * plane + q * 4)
                                       : f4{0.f, 0.f, 0.f, 0.f};
    if constexpr (SNK) {  // Snake_out at load (parameters uniform across the wave)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (k0 + u >= nk) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = (k0 + u) * 16 + q * 4;
          const f4 sc = *reinterpret_cast<const f4*>(a.s_scale + ch);
          const f4 sh = *reinterpret_cast<const f4*>(a.s_h + ch);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[u][q][e] = snake_f32(x[u][q][e], sc[e], sh[e]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u >= nk) break;
#pragma unroll
      for (int oc = 0; oc < NOUT; ++oc)
#pragma unroll
        for (int j = 0; j < 7; ++j) {
          const float* wj = a.w + (oc * 7 + j) * C + (k0 + u) * 16;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f4 w = *reinterpret_cast<const f4*>(wj + q * 4);
            z[oc][j] = fmaf(w[0], x[u][q][0], z[oc][j]);
            z[oc][j] = fmaf(w[1], x[u][q][1], z[oc][j]);
            z[oc][j] = fmaf(w[2], x[u][q][2], z[oc][j]);
            z[oc][j] = fmaf(w[3], x[u][q][3], z[oc][j]);
          }
        }
    }
  }
  const int o = f;
  const bool store = lane >= P && lane < P + kHeadOut && o < hi;
#pragma unroll
  for (int oc = 0; oc < NOUT; ++oc) {
    float y = a.bias[oc];
#pragma unroll
    for (int j = 0; j < 7; ++j) {
      const int src = min(max(lane + j - P, 0), 63);
      y += __shfl(z[oc][j], src);
    }
    if (store) a.pcm[a.rows.dst[r] + oc * a.ch_stride - lo + o] = a.no_tanh ? y : tanhf(y);
  }
}

// ------------------------------------------------------------------ tanh
// The decoder's last step, tanh after conv_out (minimaxmusic.cpp
// ARCHITECTURE, "Flow VAE"), as a pass of its own over the stored pcm: the
// split tanh ablation, which measures what folding it into the head saves.
// Four consecutive samples per thread, 16-byte loads and stores, the ragged
// end element by element; the same tanhf of the same fp32 sums as the head.
__global__ __launch_bounds__(256) void tanh_kernel(float* x, int64_t n) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 4 <= n) {
    f4 v = *reinterpret_cast<const f4*>(x + i);
    v[0] = tanhf(v[0]);
    v[1] = tanhf(v[1]);
    v[2] = tanhf(v[2]);
    v[3] = tanhf(v[3]);
    *reinterpret_cast<f4*>(x + i) = v;
  } else {
    for (int64_t j = i; j < n; ++j) x[j] = tanhf(x[j]);
  }
}

hipError_t launch_tanh(float* x, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 1023) / 1024;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tanh_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, x, n);
  return hipGetLastError();
}

hipError_t launch_head(const HeadArgs& a, hipStream_t s) {
  // keep ranges lie inside the allocated frames; the grid covers them.
  const int waves = (a.T + kHeadOut - 1) / kHeadOut;
  const dim3 grid(static_cast<unsigned>((waves + 3) / 4), static_cast<unsigned>(a.nrows));
  if (a.nout == 2 && a.s_scale)
    hipLaunchKernelGGL((head_kernel<2, 1>), grid, dim3(256), 0, s, a);
  else if (a.nout == 2)
    hipLaunchKernelGGL((head_kernel<2, 0>), grid, dim3(256), 0, s, a);
  else if (a.s_scale)
    hipLaunchKernelGGL((head_kernel<1, 1>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((head_kernel<1, 0>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------ af snake
// Alias-free Snake (TensorSharp minimax-h3 page, audio VAE: every
// nonlinearity between a 2x upsample and a 2x downsample; the 12-tap
// low-pass and its phases are described with AfArgs).  A thread owns four
// channels of one 16-channel chunk and a run of kAfRun consecutive output
// frames.  Output t sums fd[j] v[2t-5+j], j = 0 .. 11, over the activated
// 2x-rate samples v; the samples v[2t+7], v[2t+8] that output t+1 adds both
// come from input frames x[t+1 .. t+6].  A run warms up on x[t0-5 .. t0+5]
// (twelve samples) and then slides: per frame one new input frame, two
// upsampled samples of six taps, two Snakes.  It keeps no samples, only the
// six outputs they feed, partially summed: each new pair is added to
// outputs t+1 .. t+6 with their taps, after which output t+1 is complete.
// Every output thus sums its twelve terms in tap order from zero with FMAs,
// whichever run computes it, so tiles and windows of a clip give the same
// bits as the whole clip.
// Edges without branches: input frames outside [0, len) repeat the edge
// frame (clamped loads; the upsampler's replicate padding), and a 2x-rate
// sample past either end repeats the edge sample (the downsampler's): one
// select per sample (v[n < 0] = v[0], which only a run starting at frame 0
// meets, as its sixth warm-up sample; v[n > 2 len - 1] = the previous
// sample).  Lanes 4k .. 4k+3 read one 64-byte frame row; the 16 runs of a
// wave sit kAfRun frames apart, each walking its rows' cache lines in order.
#ifndef VOC_AF_RUN
#define VOC_AF_RUN 16
#endif
#ifndef VOC_AF_CPT
#define VOC_AF_CPT 4
#endif
constexpr int kAfRun = VOC_AF_RUN;
constexpr int kAfCpt = VOC_AF_CPT;  // channels per thread (2 or 4)
#ifndef VOC_AF_PREFETCH
#define VOC_AF_PREFETCH 1
#endif
#ifndef VOC_AF_MIN_WAVES
#define VOC_AF_MIN_WAVES 4  // launch bound: fewest waves per SIMD the registers must allow
#endif
constexpr int kAfPrefetch = VOC_AF_PREFETCH;  // input frames requested ahead of their use

template <int N> struct AfVec;
template <> struct AfVec<2> {
  typedef float T __attribute__((ext_vector_type(2)));
  typedef _Float16 H __attribute__((ext_vector_type(2)));
  static __device__ __forceinline__ void store_bf16(uint16_t* p, T y) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(y[0], y[1]);
  }
};
template <> struct AfVec<4> {
  typedef f4 T;
  typedef _Float16 H __attribute__((ext_vector_type(4)));
  static __device__ __forceinline__ void store_bf16(uint16_t* p, T y) {
    uint2 v;
    v.x = pack_bf16x2(y[0], y[1]);
    v.y = pack_bf16x2(y[2], y[3]);
    *reinterpret_cast<uint2*>(p) = v;
  }
};

// H16: the input (the residual stream, or conv1's output in its layout) holds
// fp16 elements.  An OUT_OP == OP_F32 output is fp32 (the head's input).
template <int OUT_OP, int H16>
__global__ __launch_bounds__(256, VOC_AF_MIN_WAVES) void af_snake_kernel(const AfArgs a) {
  typedef typename AfVec<kAfCpt>::T fv;
  typedef typename AfVec<kAfCpt>::H hv;
  constexpr int LPR = 16 / kAfCpt;   // lanes per 64-byte frame row
  constexpr int RPW = 256 / LPR;     // runs per workgroup
  const int r = blockIdx.y;
  const int nchunk = a.C / 16;
  const int chunk = blockIdx.x % nchunk;
  const int run = (blockIdx.x / nchunk) * RPW + static_cast<int>(threadIdx.x) / LPR;
  const int q = threadIdx.x % LPR;
  const int len = min(a.row_len[r] * a.rate, a.T);
  const int t0 = run * kAfRun;
  if (t0 >= len) return;
  const int c = chunk * 16 + q * kAfCpt;
  const int64_t xp = (static_cast<int64_t>(r) * a.C + chunk * 16) * a.T + q * kAfCpt;
  const fv sc = *reinterpret_cast<const fv*>(a.scale + c);
  const fv hh = *reinterpret_cast<const fv*>(a.hh + c);
  // Output element index of frame 0 of this thread's channels.
  const int64_t orow = OUT_OP == OP_F32 ? (static_cast<int64_t>(r) * a.C + chunk * 16) * a.T + q * kAfCpt
                                        : (static_cast<int64_t>(r) * a.C + (c / 32) * 32) * a.T + c % 32;
  char* obase = static_cast<char*>(a.out);
  const int n_last = 2 * len - 1;
  const fv zero = fv(0.f);
  auto ld = [&](int t) -> fv {
    t = min(max(t, 0), len - 1);
    const int64_t i = xp + static_cast<int64_t>(t) * kHChunk;
    if constexpr (H16)
      return __builtin_convertvector(*reinterpret_cast<const hv*>(reinterpret_cast<const _Float16*>(a.x) + i), fv);
    else
      return *reinterpret_cast<const fv*>(a.x + i);
  };
  auto snake_v = [&](fv u) -> fv {
    fv v;
#pragma unroll
    for (int e = 0; e < kAfCpt; ++e) v[e] = snake_f32(u[e], sc[e], hh[e]);
    return v;
  };
  auto pick = [](bool cond, fv x, fv y) -> fv {  // cond ? x : y, per element
    fv o;
#pragma unroll
    for (int e = 0; e < kAfCpt; ++e) o[e] = cond ? x[e] : y[e];
    return o;
  };
  auto store = [&](int t, fv y) {
    if constexpr (OUT_OP == OP_F32)
      *reinterpret_cast<fv*>(reinterpret_cast<float*>(obase) + orow + static_cast<int64_t>(t) * 16) = y;
    else
      AfVec<kAfCpt>::store_bf16(reinterpret_cast<uint16_t*>(obase) + orow + static_cast<int64_t>(t) * 32, y);
  };
  // A[k] collects output t + k (t = t0 at the start).
  fv A[6];
#pragma unroll
  for (int k = 0; k < 6; ++k) A[k] = zero;
  fv R[6];
  fv vlast;
  {
    // Warm-up.  X[k] = x[t0 - 5 + k]; sample i is v[n], n = 2 t0 - 5 + i:
    //   i odd  (n = 2m,   m = t0 + (i - 5) / 2): fe taps on X[(i - 1) / 2 .. + 5]
    //   i even (n = 2m+1, m = t0 + (i - 6) / 2): fo taps on X[i / 2 .. + 5]
    fv X[11];
#pragma unroll
    for (int k = 0; k < 11; ++k) X[k] = ld(t0 - 5 + k);
    auto sample = [&](int i) -> fv {
      const int b = (i & 1) ? (i - 1) / 2 : i / 2;
      fv u = zero;
#pragma unroll
      for (int k = 0; k < 6; ++k) u += ((i & 1) ? a.fe[k] : a.fo[k]) * X[b + k];
      return snake_v(u);
    };
    const fv v5 = sample(5);  // v[2 t0]: v[0] for the run that starts the row
    vlast = v5;
#pragma unroll
    for (int i = 0; i < 12; ++i) {
      const int n = 2 * t0 - 5 + i;
      fv v = i == 5 ? v5 : sample(i);
      v = pick(n < 0, v5, v);
      v = pick(n > n_last, vlast, v);
      vlast = v;
#pragma unroll
      for (int k = 0; k < 6; ++k)
        if (i - 2 * k >= 0) A[k] += a.fd[i - 2 * k] * v;  // tap i - 2k of output t0 + k
    }
#pragma unroll
    for (int k = 0; k < 5; ++k) R[k] = X[6 + k];
  }
  fv nx[kAfRun];  // nx[s] = x[t0 + s + 6]
#pragma unroll
  for (int s = 0; s < kAfPrefetch; ++s) nx[s] = ld(t0 + s + 6);
#pragma unroll
  for (int s = 0; s < kAfRun; ++s) {
    const int t = t0 + s;
    if (s + kAfPrefetch < kAfRun - 1) nx[s + kAfPrefetch] = ld(t + kAfPrefetch + 6);
    if (t < len) store(t, A[0]);
    if (s + 1 < kAfRun) {
      R[5] = nx[s];
      fv uo = zero, ue = zero;
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        uo += a.fo[k] * R[k];  // v[2t + 7]
        ue += a.fe[k] * R[k];  // v[2t + 8]
      }
      const fv vo = pick(2 * t + 7 > n_last, vlast, snake_v(uo));
      const fv ve = pick(2 * t + 8 > n_last, vo, snake_v(ue));
      vlast = ve;
#pragma unroll
      for (int k = 0; k < 5; ++k) A[k] = A[k + 1];
      A[5] = zero;
#pragma unroll
      for (int k = 0; k < 6; ++k) {  // output t + 1 + k: taps 10 - 2k and 11 - 2k
        A[k] += a.fd[10 - 2 * k] * vo;
        A[k] += a.fd[11 - 2 * k] * ve;
      }
#pragma unroll
      for (int k = 0; k < 5; ++k) R[k] = R[k + 1];
    }
  }
}

hipError_t launch_af_snake(const AfArgs& a, hipStream_t s) {
  constexpr int RPW = 256 / (16 / kAfCpt);
  const int runs = (a.T + kAfRun - 1) / kAfRun;
  const dim3 grid(static_cast<unsigned>((a.C / 16) * ((runs + RPW - 1) / RPW)), static_cast<unsigned>(a.rows));
  if (a.out_op == OP_F32 && a.h16)
    hipLaunchKernelGGL((af_snake_kernel<OP_F32, 1>), grid, dim3(256), 0, s, a);
  else if (a.out_op == OP_F32)
    hipLaunchKernelGGL((af_snake_kernel<OP_F32, 0>), grid, dim3(256), 0, s, a);
  else if (a.h16)
    hipLaunchKernelGGL((af_snake_kernel<OP_BF16, 1>), grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;  // bf16 operands always come with an fp16 residual stream
  return hipGetLastError();
}

// ------------------------------------------------------- plain Snake
// The standalone elementwise Snake (an ablation: the decoder normally
// applies Snake in the producer's epilogue or the consumer's staging).  A
// thread handles one 16-byte unit of one output frame row: four fp32
// channels, or eight bf16 channels (read from two fp32 units).  A wave
// covers 16 consecutive frames of an output chunk, so reads and writes are
// whole 64-byte rows.
template <int OUT_OP, int H16>
__global__ __launch_bounds__(256) void snake_kernel(const AfArgs a) {
  constexpr int CH = OUT_OP == OP_F32 ? 16 : 32;  // channels per output row
  constexpr int CPT = CH / 4;                     // channels per thread
  const int r = blockIdx.y;
  const int nchunk = a.C / CH;
  const int chunk = blockIdx.x % nchunk;
  const int t = (blockIdx.x / nchunk) * 64 + static_cast<int>(threadIdx.x >> 2);
  const int q = threadIdx.x & 3;
  const int len = min(a.row_len[r] * a.rate, a.T);
  if (t >= len) return;
  const int c = chunk * CH + q * CPT;  // first channel of this thread
  f4 y[CPT / 4];
#pragma unroll
  for (int k = 0; k < CPT / 4; ++k) {
    const int ck = c + 4 * k;
    const f4 x = load_h4<H16>(a.x, (static_cast<int64_t>(r) * a.C + (ck & ~15)) * a.T +
                                        static_cast<int64_t>(t) * kHChunk + (ck & 15));
    const f4 sc = *reinterpret_cast<const f4*>(a.scale + ck);
    const f4 hh = *reinterpret_cast<const f4*>(a.hh + ck);
#pragma unroll
    for (int e = 0; e < 4; ++e) y[k][e] = snake_f32(x[e], sc[e], hh[e]);
  }
  const int64_t idx = (static_cast<int64_t>(r) * a.C + chunk * CH) * a.T + static_cast<int64_t>(t) * CH + q * CPT;
  if constexpr (OUT_OP == OP_F32) {
    store_h4<OP_F32>(a.out, idx, y[0]);  // fp32: the head's input (or fp32 operands)
  } else {
    uint4 v;
    v.x = pack_bf16x2(y[0][0], y[0][1]);
    v.y = pack_bf16x2(y[0][2], y[0][3]);
    v.z = pack_bf16x2(y[1][0], y[1][1]);
    v.w = pack_bf16x2(y[1][2], y[1][3]);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + idx) = v;
  }
}

hipError_t launch_snake(const AfArgs& a, hipStream_t s) {
  const int ch = a.out_op == OP_F32 ? 16 : 32;
  const dim3 grid(static_cast<unsigned>((a.C / ch) * ((a.T + 63) / 64)), static_cast<unsigned>(a.rows));
  if (a.out_op == OP_F32 && a.h16)
    hipLaunchKernelGGL((snake_kernel<OP_F32, 1>), grid, dim3(256), 0, s, a);
  else if (a.out_op == OP_F32)
    hipLaunchKernelGGL((snake_kernel<OP_F32, 0>), grid, dim3(256), 0, s, a);
  else if (a.h16)
    hipLaunchKernelGGL((snake_kernel<OP_BF16, 1>), grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;  // bf16 operands always come with an fp16 residual stream
  return hipGetLastError();
}

// ----------------------------------------------------------- col2im
// The overlap-add half of a ConvTranspose1d computed as GEMM + col2im (the
// pages' GGML lowering, kept as an ablation of the polyphase GEMM; qwentts.cpp
// ARCHITECTURE, "Custom GGML ops").  With K = 2s every output frame tau
// gathers exactly two products: k = (tau + crop) mod s at input frame
// n = (tau + crop) / s, and k + s at n - 1.  A thread handles four channels
// of one output frame (whole 64-byte rows per wave).
template <int OP>
__global__ __launch_bounds__(256) void col2im_kernel(const Col2imArgs a) {
  const int r = blockIdx.y;
  const int nchunk = a.Cout / 16;
  const int chunk = blockIdx.x % nchunk;
  const int tau = (blockIdx.x / nchunk) * 64 + static_cast<int>(threadIdx.x >> 2);
  const int q = threadIdx.x & 3;
  const int lin = min(a.row_len[r] * a.rate_in, a.T_col);
  const int lout = min(a.row_len[r] * a.rate_in * a.s, a.T_out);
  if (tau >= lout) return;
  const int o = chunk * 16 + q * 4;
  const int mcol = 2 * a.s * a.Cout;
  // The column matrix is in the residual-stream layout of the column GEMM's
  // output (fp16 elements for bf16 operands).
  const int64_t colr = static_cast<int64_t>(r) * mcol * a.T_col;
  auto z = [&](int k, int n) -> f4 {  // z[k*Cout + o .. + 3][n]
    const int m = k * a.Cout + o;
    return load_h4<OP>(a.col, colr + static_cast<int64_t>(m & ~15) * a.T_col +
                                  static_cast<int64_t>(n) * kHChunk + (m & 15));
  };
  const int n = (tau + a.crop) / a.s, k = tau + a.crop - n * a.s;
  f4 v = *reinterpret_cast<const f4*>(a.bias + o);
  if (n < lin) v += z(k, n);
  if (n >= 1 && n - 1 < lin) v += z(k + a.s, n - 1);
  if (a.s_out) v = round_h4<OP>(v);  // the Snake below starts from the stored h
  if (a.h_out)
    store_h4<OP>(a.h_out, (static_cast<int64_t>(r) * a.Cout + chunk * 16) * a.T_out +
                              static_cast<int64_t>(tau) * kHChunk + q * 4, v);
  if (a.s_out) {
    if (a.s_alpha) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = snake_f32(v[e], a.s_alpha[o + e], a.s_invden[o + e]);
    }
    constexpr int CH = OP == OP_F32 ? 16 : 32;
    store_op4<OP>(a.s_out, (static_cast<int64_t>(r) * a.Cout + (o / CH) * CH) * a.T_out +
                               static_cast<int64_t>(tau) * CH + o % CH, v);
  }
}

hipError_t launch_col2im(const Col2imArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.Cout / 16) * ((a.T_out + 63) / 64)), static_cast<unsigned>(a.rows));
  if (a.op == OP_F32)
    hipLaunchKernelGGL(col2im_kernel<OP_F32>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(col2im_kernel<OP_BF16>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- copy
// A plain copy that keeps kCopyU independent 16-byte loads in flight per
// thread: a workgroup moves chunks of 256 * kCopyU units, its loads all
// issued before its stores, with non-temporal hints (the data is touched
// once).  One chunk per workgroup over the whole buffer.  Measured on
// MI355X over 1 GiB: 6.3 TB/s counting bytes read and written, against
// 4.6 TB/s for one load per thread on a capped grid and 5.8 TB/s without
// the hints.
constexpr int kCopyU = 4;

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_kernel(u4v* dst, const u4v* src, int64_t n) {
  const int64_t step = static_cast<int64_t>(gridDim.x) * 256 * kCopyU;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * 256 * kCopyU + threadIdx.x; base < n; base += step) {
    u4v v[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const int64_t i = base + u * 256;
      if (i < n) v[u] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const int64_t i = base + u * 256;
      if (i < n) __builtin_nontemporal_store(v[u], dst + i);
    }
  }
}

hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  int64_t blocks = (n + 256 * kCopyU - 1) / (256 * kCopyU);
  if (blocks > 0x7fffffff) blocks = 0x7fffffff;  // then the grid-stride loop covers the rest
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(copy_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<u4v*>(dst), static_cast<const u4v*>(src), n);
  return hipGetLastError();
}

}  // namespace voc
