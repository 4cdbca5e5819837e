// host_config.h -- host-only parts of libvocoder: configuration checks, the
// exact tiling halos, the GEMM plane limit, window bookkeeping, the checkpoint
// tensor table and the alias-free Snake's low-pass design.  Plain C++17 with
// no HIP dependency, so that it also builds with g++ under the address and
// undefined-behaviour sanitizers.
#pragma once
#include <stdint.h>

#include <map>
#include <string>
#include <vector>

#include "../../include/vocoder.h"

namespace voc {

constexpr int kChunkBytes = 64;
constexpr int kHChunk = 16;  // residual stream channels per chunk row
// Bytes per residual-stream element: fp32 for fp32 operands, fp16 for bf16.
constexpr int h_size(int op) { return op == 0 ? 4 : 2; }
constexpr int kAfTaps = 12;  // taps of the alias-free Snake's low-pass

enum OpType { OP_F32 = 0, OP_BF16 = 1 };

// Frames per workgroup of the fused residual-unit kernel for width C (0: no
// fused instance); defined with the kernels.
int res_unit_tile(int op, int C, bool big, int terms = 1);

int total_stride(const voc_config& c);
voc_status validate(const voc_config* c, std::string* why);
int64_t floordiv(int64_t a, int64_t b);
void compute_halos(const voc_config& c, int* h_left, int* h_right);
int compute_halo(const voc_config& c);

// The GEMM plane limit (buffer loads with 32-bit byte offsets).
extern const int64_t kPlaneLimitBytes;
extern const int64_t kStreamCtxMax;
bool gemm_plane_ok(int64_t plane_frames, int64_t lb, int64_t S);
int64_t gemm_rate_max(const voc_config& g, int op, bool units_unfused);
int64_t max_row_frames(const voc_config& g, int op, bool units_unfused);

// Window stitching bookkeeping.
void window_keep(int64_t k, int64_t n, int64_t L, int64_t L_last, int64_t cl, int64_t cr, int64_t* lo,
                 int64_t* hi);
bool windows_valid(int64_t n, int64_t L, int64_t L_last, int64_t cl, int64_t cr);

// Checkpoint tensors: name -> squeezed shape (size-1 dims removed).
struct Expect {
  std::vector<int64_t> shape;
};
std::vector<int64_t> squeeze(const int64_t* shape, int nd);
std::map<std::string, Expect> expected_tensors(const voc_config& g);
bool all_finite(const float* p, int64_t n);
int64_t numel(const voc_tensor& t);

// The alias-free Snake's 12-tap low-pass: upsampler polyphase taps fe, fo
// (gain 2) and the downsampler taps fd.
double bessel_i0(double x);
void design_af_filter(float* fe, float* fo, float* fd);

}  // namespace voc
