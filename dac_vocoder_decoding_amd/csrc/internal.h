// internal.h -- device-side data layouts and kernel launch interfaces of
// libvocoder (not part of the public ABI).
//
// Activation layouts in HBM ("channel-chunked channels-last"):
//   operand tensors (matrix-core inputs, fp32 or bf16):
//       [row][C / CH][T][CH] with CH = 64 bytes / element size
//       (16 fp32 or 32 bf16 channels per chunk)
//   residual stream h: [row][C / 16][T][16], fp32 elements with fp32
//       operands, fp16 elements with bf16 operands (arithmetic on h is fp32;
//       the float* members below then point at fp16 data)
// One 64-byte chunk row holds CH consecutive channels of one time frame, so a
// GEMM tile of a channel chunk over consecutive frames is one contiguous span.
//
// Packed conv weights (matrix-core dtype): [Cin / CH][tap][M][CH]
//   Conv1d  (Cout, Cin, K):  tap = k,           M = Cout, m = o
//   ConvT   (Cin, Cout, 2s): tap t in {0,1},    M = s*Cout, m = r*Cout + o,
//                            value w[i][o][t*s + r]   (polyphase split)
// Head weights: fp32 [out channel][k][C] (bf16-rounded values for BF16 configs).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "host_config.h"  // kChunkBytes, kHChunk, OpType, kAfTaps, res_unit_tile

namespace voc {

inline int op_chunk(int op) { return op == OP_F32 ? 16 : 32; }
inline int op_size(int op) { return op == OP_F32 ? 4 : 2; }

// Per-row metadata of one decode (device arrays, length = rows).
struct RowInfo {
  const int* len;       // valid latent frames of the row
  const int* src_b;     // source batch row of the latent
  const int* start;     // first latent frame of the row in the source
  const int* keep_lo;   // first output sample kept (row-local)
  const int* keep_hi;   // one past the last output sample kept
  const int64_t* dst;   // pcm element offset of the first kept sample
};

// One implicit-GEMM convolution launch:
//   acc[n][m] = sum_tap sum_i W[tap][m][i] * X[row][n + off0 + tap*offstep][i]
// X frames outside [0, len*rate_in) read as zero.  Output frame
// tau = n*ups + m / Cout - crop, channel o = m % Cout, kept if
// 0 <= tau < min(len*rate_out, T_out).
// Epilogue: v = acc + bias[o] (+ res); h_out <- v (fp32);
//           s_out <- Snake(v; s_alpha, s_invden) in the operand dtype
//           (v itself when s_alpha is null).
struct ConvArgs {
  const void* x;
  int T_in;       // allocated frames per row of x
  int Cin;
  const int* row_len;
  int rate_in, rate_out;
  const void* w;
  int M, Cout;
  int off0, offstep, min_off, halo;
  int N;          // GEMM positions per row
  int n_tiles, m_tiles, rows;
  int m_fast;     // tile order: 1 = the M-tiles of one N-range are adjacent, 0 = N fastest
  const float* bias;
  float* h_out;
  const float* res;
  void* s_out;
  const float* s_alpha;
  const float* s_invden;
  const float* hs_scale;  // if set, h_out receives Snake(v) with these
  const float* hs_h;      // parameters instead of v (the head's Snake)
  int T_out, ups, crop;
  int lb;         // frames in [-lb, 0) of x are read from memory (a stream's context), else zero
  int in_stride;  // > 1: strided conv (2 taps); GEMM frame m of virtual chunk c reads input row
                  // m * s + c % s - s/2 of chunk c / s, s = in_stride (Cin counts real channels)
  int two_term;   // 1 (bf16): a decoder with two-term operands: s_out holds both terms,
                  // [row][2 * Cout / CH][T][CH] with the low terms in channel planes Cout / CH..,
                  // and res / h_out hold fp32 elements (its residual stream is fp32)
};

// Tile shape families of the conv GEMM kernel.
enum ConvVariant {
  CV_128x256 = 0,
  CV_64x256 = 1,
  CV_96x256 = 2,
  CV_128x128 = 3,
  CV_64x128 = 4,
  CV_192x128 = 5,
  CV_16x128 = 6,   // narrow-M tiles for the k=7 convs of 16- and 32-channel units
  CV_32x128 = 7,
  CV_COUNT = 8
};
int conv_variant_bm(int v);
int conv_variant_bn(int v);
bool conv_variant_ok(int v, int taps);

// tag: 1 conv_in / dec_in_proj, 3 the encoder's conv_out / projection, else
// 0 (separate kernel names for profilers; the strided conv picks its own).
hipError_t launch_conv(int op, int taps, int variant, int tag, const ConvArgs& a, hipStream_t s);

// One fused residual unit over all C channels of BN-frame tiles:
//   h <- h_in + conv2(Snake2(conv1_dil(x) + b1)) + b2;  s_out <- Snake_next(h).
// x is Snake1(h_in) in the operand dtype: read from the operand tensor x, or
// (x_from_h) computed in the kernel from h_in with the a1 parameters, in
// which case h must be a different buffer from h_in.  Same layouts as ConvArgs.
struct ResUnitArgs {
  const void* x;         // unused when x_from_h
  int x_from_h;
  const float* a1_scale;  // Snake1: alpha/pi, 1/(2 den) (x_from_h only)
  const float* a1_h;
  const float* h_in;     // residual stream read (equal to h unless x_from_h)
  int T, C;
  const int* row_len;
  int rate, dil;
  const void* w1;        // packed [C/CH][7][C][CH]
  const float* b1;
  const float* a2_scale;  // Snake2: alpha/pi, 1/(2 den)
  const float* a2_h;
  const void* w2;        // packed [C/CH][1][C][CH]
  const float* b2;
  float* h;              // residual stream written
  int terms;             // 1, or 2 (bf16): two-term operands (x / s_out planes [row][2C/CH][T][CH],
                         // w1 / w2 with every channel chunk plane present twice); 0 counts as 1
  int store_h;           // 0: the updated h is not stored (nothing reads it)
  void* s_out;           // may be null
  const float* s_scale;
  const float* s_h;
  const float* hs_scale;  // if set, h receives Snake(h) (the head's Snake)
  const float* hs_h;
  int pad;               // conv1 left padding: 3*dil ("same") or 6*dil (causal)
  int lb;                // frames in [-lb, 0) of the input are read from memory, else zero
  int n_tiles, rows;
};
// res_unit_tile(op, C, big) (host_config.h): frames per workgroup of the
// fused kernel for width C, or 0 if there is no fused instance for (op, C);
// big selects the large-frame tile of that width (0 if it has none).
// Whether units of width C run with x_from_h (Snake1 computed in the kernel).
hipError_t launch_res_unit(int op, const ResUnitArgs& a, bool big, hipStream_t s);

// Weight-norm fold + cast + repack, one workgroup per axis-0 slice.
enum PackKind { PACK_CONV = 0, PACK_CONVT = 1, PACK_HEAD = 2, PACK_DOWN = 3 };
struct FoldArgs {
  const float* v;
  const float* g;   // null: no weight norm (w = v)
  int64_t d0, rest;
  int kind;
  int op;           // operand dtype of the packed output (head: always fp32 storage)
  int round_bf16;   // head of a BF16 config: round to bf16, store as fp32
  int cin, cout, k, stride;  // original tensor geometry
  void* out;
  double* norms;    // [d0]
};
hipError_t launch_fold(const FoldArgs& a, hipStream_t s);

// Latent / stage import: x fp32 [src_b][C][T_src] -> per output row r:
//   frames [0, T) from source frames start[r] + t (t < len[r], else zero);
//   s_out (operand dtype, chunked, optional Snake), h_out (fp32 chunked).
struct ImportArgs {
  const float* x;
  int64_t T_src;
  int C;
  RowInfo rows;
  int nrows;
  int T;            // allocated frames per output row (plane length)
  int T_write;      // frames written per row (0: T)
  int op;
  void* s_out;      // may be null
  const float* s_alpha;  // null -> identity
  const float* s_invden;
  float* h_out;     // may be null
  const float* h_scale;  // if set, h_out receives Snake(x) with these parameters
  const float* h_h;
};
hipError_t launch_import(const ImportArgs& a, hipStream_t s);

// Mono audio x fp32 [rows][T] -> operand [rows][1][T][CH] with channel 0 = x.
hipError_t launch_audio_import(int op, const float* x, void* out, int64_t T, int rows, hipStream_t s);

// h fp32 chunked [rows][C/16][T][16] -> y fp32 [rows][C][T].
hipError_t launch_export(int op, const void* h, float* y, int rows, int C, int T, hipStream_t s);

// Head: pcm[dst[r] + o * ch_stride + tau - keep_lo[r]] = tanh(bias[o] +
//   sum_j sum_i w[o][j][i] * sh[r][tau + j - pad][i]) for tau in
// [keep_lo[r], keep_hi[r]) and output channel o < nout, where sh is
// Snake_out(h), already applied by the producer (the last residual unit's
// epilogue, or the alias-free Snake kernel).
struct HeadArgs {
  const float* h;   // Snake_out(h) in fp32, or with s_scale set the fp16 residual stream h
  const float* s_scale;  // Snake_out parameters (alpha / pi, 1 / (2 den)) applied at load,
  const float* s_h;      // or null
  int C, T;         // channels, allocated frames per row
  RowInfo rows;
  int nrows;
  int rate;         // frames per latent frame
  int pad;          // left padding of the k=7 conv: 3 ("same") or 6 (causal)
  int lb;           // frames in [-lb, 0) of h are read from memory, else zero
  int nout;         // output channels (1 or 2)
  int64_t ch_stride;  // pcm elements between the output channels of a row
  const float* w;   // [nout][7][C]
  float bias[2];
  float* pcm;
  int no_tanh;      // 1: store the pre-tanh sum (the split tanh ablation)
};
hipError_t launch_head(const HeadArgs& a, hipStream_t s);

// x[i] = tanh(x[i]) for i < n, in place (x 16-byte aligned).
hipError_t launch_tanh(float* x, int64_t n, hipStream_t s);

hipError_t launch_copy(void* dst, const void* src, int64_t bytes, hipStream_t s);

// Matrix-core loop microbenchmark: mfma_loop_blocks() workgroups of 256
// threads each run `iters` iterations of independent MFMA chains of the
// operand dtype op; out receives one float per thread.
int mfma_loop_blocks();
double mfma_loop_flops(int op, int64_t iters);
hipError_t launch_mfma_loop(int op, int64_t iters, float* out, hipStream_t s);
// The same with 32x32 MFMAs (fp32 32x32x2, bf16 32x32x16).
double mfma32_loop_flops(int op, int64_t iters);
hipError_t launch_mfma32_loop(int op, int64_t iters, float* out, hipStream_t s);

// Alias-free Snake over a residual-stream tensor (fp32 chunked, 16 channels
// per 64-byte frame row): per row r with valid frames [0, len), len =
// min(row_len[r] * rate, T),
//   u = up2(x)   x replicate-padded;  u[2m]   = sum_k fe[k] x[m - 3 + k],
//                                      u[2m+1] = sum_k fo[k] x[m - 2 + k]
//   v = Snake(u) (scale, hh as for every Snake)
//   y[t] = sum_j fd[j] v[2t - 5 + j]   v replicate-padded over [0, 2 len)
// written for t < len to out in the out_op layout (fp32 16-channel chunks,
// or bf16 32-channel chunks).  fe[k] = 2 f[11 - 2k], fo[k] = 2 f[10 - 2k],
// fd = f (the 12-tap low-pass).
struct AfArgs {
  const float* x;
  void* out;
  int out_op;
  int C, T;           // channels, allocated frames per row (plane length)
  const int* row_len;
  int rate;
  const float* scale;  // alpha / pi per channel
  const float* hh;     // 1 / (2 den) per channel
  float fe[6], fo[6], fd[kAfTaps];
  int rows;
  int h16;             // x holds fp16 elements (the bf16 decoders' residual stream)
};
hipError_t launch_af_snake(const AfArgs& a, hipStream_t s);
// col2im overlap-add of a ConvTranspose1d computed as a plain GEMM into a
// column matrix (an ablation of the polyphase GEMM): col holds, per row, the
// fp32 [2s*Cout / 16][T_col][16] products z[k*Cout + o][n] = sum_i w[i][o][k]
// x[i][n]; output frame tau, channel o receives bias[o] + z[k][n] over the
// (n, k) with n*s + k = tau + crop (two of them), then the epilogue of the
// polyphase GEMM: h_out (fp32) and/or s_out = Snake(v) in the operand dtype.
struct Col2imArgs {
  const float* col;
  int T_col;            // allocated frames per row of col
  int Cout, s, crop;
  const float* bias;
  float* h_out;
  void* s_out;
  const float* s_alpha;  // null: s_out receives v itself
  const float* s_invden;
  int T_out;            // allocated frames per row of the outputs
  const int* row_len;
  int rate_in;          // input frames per latent frame
  int rows, op;
};
hipError_t launch_col2im(const Col2imArgs& a, hipStream_t s);

// Plain Snake of the same tensors, elementwise (the filter fields unused):
// the standalone Snake stage of the split ablation.
hipError_t launch_snake(const AfArgs& a, hipStream_t s);

// Streaming: one layer's carried context.  buf points at frame 0 of the
// first plane of the layer's input; planes of plane_bytes bytes hold 64-byte
// frame rows, the chunk in frames [0, Tr) and ctx margin frames before it.
// The margin receives old_state; new_state receives the last ctx frames of
// (old_state, chunk).  States are [planes][ctx][64 bytes].
struct LayerStateArgs {
  unsigned char* buf;
  int64_t plane_bytes, planes;
  int ctx, Tr;
  int row_bytes;    // bytes per frame row of a plane: 64 (operand), or 16 residual elements
  const unsigned char* old_state;
  unsigned char* new_state;
};
hipError_t launch_layer_state(const LayerStateArgs& a, hipStream_t s);

}  // namespace voc
