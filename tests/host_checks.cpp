// Host-only checks of libvocoder's configuration validation, exact tiling
// halos, GEMM plane limit, window bookkeeping, checkpoint tensor table and
// alias-free low-pass design (dac_vocoder_decoding_amd/csrc/host_config.cpp),
// built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers.py.  No device code is involved.
#include "../dac_vocoder_decoding_amd/csrc/host_config.h"

#include <cmath>
#include <cstdio>
#include <cstring>

namespace voc {
// The fused residual-unit widths of the kernel file (fp32 16..128, bf16
// 64..192), standing in for the kernels, which this build does not contain.
int res_unit_tile(int op, int C, bool big, int /*terms*/) {
  const bool f = op == OP_F32 ? (C == 16 || C == 32 || C == 64 || C == 96 || C == 128)
                              : (C == 64 || C == 96 || C == 128 || C == 192);
  return f ? (big ? 256 : 128) : 0;
}
}  // namespace voc

using namespace voc;

static int g_fail = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #cond);     \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

static voc_config dflt() {
  voc_config c;
  voc_config_default(&c);
  return c;
}

int main() {
  voc_config c = dflt();
  EXPECT(voc_config_validate(&c) == VOC_OK);
  EXPECT(voc_config_hop(&c) == 512);
  EXPECT(voc_config_halo(&c) == 10);
  // The last ConvTranspose1d (input rate 256) bounds the default decoder.
  EXPECT(voc_config_max_frames(&c) == (((int64_t(1) << 32) - (int64_t(1) << 16)) / 64 - 566) / 256);
  EXPECT(voc_config_validate(nullptr) == VOC_INVALID_PARAMS);
  EXPECT(voc_config_halo(nullptr) == VOC_INVALID_PARAMS);

  // Invalid configurations, one field at a time.
  struct Bad { const char* what; void (*f)(voc_config*); };
  const Bad bad[] = {
      {"n_blocks 0", [](voc_config* x) { x->n_blocks = 0; }},
      {"n_blocks 9", [](voc_config* x) { x->n_blocks = 9; }},
      {"n_res 0", [](voc_config* x) { x->n_res = 0; }},
      {"kernel 5", [](voc_config* x) { x->in_kernel = 5; }},
      {"act", [](voc_config* x) { x->act = 7; }},
      {"dtype", [](voc_config* x) { x->dtype = 3; }},
      {"crop", [](voc_config* x) { x->convt_crop = 1; }},
      {"tile", [](voc_config* x) { x->tile_frames = -1; }},
      {"latent 60", [](voc_config* x) { x->latent_channels = 60; }},
      {"width 100", [](voc_config* x) { x->width[2] = 100; }},
      {"last width 1024", [](voc_config* x) { x->width[4] = 1024; }},
      {"stride 0", [](voc_config* x) { x->stride[0] = 0; }},
      {"stride 65", [](voc_config* x) { x->stride[1] = 65; }},
      {"dilation 10", [](voc_config* x) { x->dilation[1] = 10; }},
      {"log params", [](voc_config* x) { x->snake_log_params = 2; }},
      {"in_proj 24", [](voc_config* x) { x->in_proj = 24; }},
      {"causal 2", [](voc_config* x) { x->causal = 2; }},
      {"af 2", [](voc_config* x) { x->af_snake = 2; }},
      {"out 3", [](voc_config* x) { x->out_channels = 3; }},
      {"af causal", [](voc_config* x) { x->af_snake = 1; x->causal = 1; }},
      {"terms 3", [](voc_config* x) { x->operand_terms = 3; }},
      {"terms f32", [](voc_config* x) { x->operand_terms = 2; }},
      {"terms af", [](voc_config* x) { x->operand_terms = 2; x->dtype = VOC_BF16; x->af_snake = 1; }},
      {"abi", [](voc_config* x) { x->abi_version = VOC_ABI_VERSION + 1; }},
      {"hop", [](voc_config* x) { x->stride[0] = x->stride[1] = x->stride[2] = x->stride[3] = 64; }},
  };
  for (const Bad& b : bad) {
    voc_config x = dflt();
    b.f(&x);
    std::string why;
    if (validate(&x, &why) != VOC_INVALID_PARAMS || why.empty()) {
      std::fprintf(stderr, "FAIL: %s accepted\n", b.what);
      ++g_fail;
    }
    EXPECT(voc_config_hop(&x) == VOC_INVALID_PARAMS && voc_config_max_frames(&x) == VOC_INVALID_PARAMS);
  }

  // Halos: causal (left only) and alias-free stacks.
  voc_config k = dflt();
  k.causal = 1;
  int hl = 0, hr = 0;
  compute_halos(k, &hl, &hr);
  EXPECT(hl == 19 && hr == 0);
  voc_config a = dflt();
  a.af_snake = 1;
  EXPECT(compute_halo(a) == 20);

  // Plane limit: rows of the returned length fit, one more does not.
  for (int op = 0; op < 2; ++op)
    for (int unfused = 0; unfused < 2; ++unfused) {
      const int64_t m = max_row_frames(c, op, unfused != 0);
      const int64_t r = gemm_rate_max(c, op, unfused != 0);
      EXPECT(gemm_plane_ok(m * r, kStreamCtxMax, 1));
      EXPECT(!gemm_plane_ok((m + 1) * r + 512, kStreamCtxMax, 1));
      EXPECT(r == (unfused ? 512 : 256));
    }
  EXPECT(!gemm_plane_ok(-1, 0, 1));

  // Window bookkeeping: the pages' 689-frame windows with crops 86 / 258
  // keep 345 frames in the middle; each window must keep a frame.
  int64_t lo = 0, hi = 0, kept = 0;
  for (int64_t w = 0; w < 5; ++w) {
    window_keep(w, 5, 689, 683, 86, 258, &lo, &hi);
    EXPECT(hi > lo);
    kept += hi - lo;
  }
  EXPECT(kept == (689 - 258) + 3 * 345 + (683 - 86));
  EXPECT(windows_valid(5, 689, 683, 86, 258));
  EXPECT(!windows_valid(3, 100, 100, 50, 50));
  EXPECT(!windows_valid(0, 10, 10, 0, 0) && !windows_valid(2, 10, 11, 0, 0) && !windows_valid(2, 10, 10, -1, 0));
  EXPECT(windows_valid(1, 10, 4, 0, 0));

  // Checkpoint table of the default decoder: conv_in, 4 blocks of a Snake,
  // a ConvTranspose1d and 3 units (2 Snakes, 2 convs), snake_out, conv_out.
  const auto t = expected_tensors(c);
  EXPECT(t.size() == 3 + 4 * (1 + 3 + 3 * (2 + 6)) + 1 + 3);
  EXPECT(t.at("blocks.0.conv_t1.weight_v").shape == (std::vector<int64_t>{1024, 512, 16}));
  EXPECT(t.at("conv_out.weight_v").shape == (std::vector<int64_t>{64, 7}));   // size-1 dims squeezed
  const int64_t sh[4] = {1, 64, 1, 1};
  EXPECT(squeeze(sh, 4) == std::vector<int64_t>{64});
  float v[3] = {1.f, NAN, 2.f};
  EXPECT(!all_finite(v, 3) && all_finite(v, 1));

  // Low-pass: unit DC gain, symmetric, each polyphase half sums to 1.
  float fe[6], fo[6], fd[kAfTaps];
  design_af_filter(fe, fo, fd);
  double sd = 0.0, se = 0.0, so = 0.0;
  for (int i = 0; i < kAfTaps; ++i) sd += fd[i];
  for (int i = 0; i < 6; ++i) se += fe[i], so += fo[i];
  EXPECT(std::fabs(sd - 1.0) < 1e-6 && std::fabs(se - 1.0) < 1e-6 && std::fabs(so - 1.0) < 1e-6);
  for (int i = 0; i < kAfTaps; ++i) EXPECT(fd[i] == fd[kAfTaps - 1 - i]);
  EXPECT(std::fabs(bessel_i0(0.0) - 1.0) < 1e-15 && std::fabs(bessel_i0(1.0) - 1.2660658777520082) < 1e-14);

  // A deterministic sweep of configurations through validation, halos and
  // the plane limit (exercises the host paths under the sanitizers).
  uint64_t s = 0x9E3779B97F4A7C15ull;
  auto rnd = [&](int n) { s = s * 6364136223846793005ull + 1442695040888963407ull; return int((s >> 33) % n); };
  int valid = 0;
  for (int it = 0; it < 3000; ++it) {
    voc_config x = dflt();
    x.n_blocks = 1 + rnd(4);
    for (int b = 0; b <= x.n_blocks; ++b) x.width[b] = 16 * (1 + rnd(40));
    for (int b = 0; b < x.n_blocks; ++b) x.stride[b] = 1 + rnd(8);
    x.n_res = 1 + rnd(4);
    for (int r = 0; r < x.n_res; ++r) x.dilation[r] = 1 + rnd(9);
    x.causal = rnd(2);
    x.af_snake = x.causal ? 0 : rnd(2);
    x.dtype = rnd(2);
    x.act = rnd(2);
    x.out_channels = 1 + rnd(2);
    if (voc_config_validate(&x) != VOC_OK) continue;
    ++valid;
    int l = -1, r = -1;
    compute_halos(x, &l, &r);
    EXPECT(l >= 0 && r >= 0 && (!x.causal || r == 0));
    EXPECT(voc_config_max_frames(&x) > 0);
    EXPECT(expected_tensors(x).size() > 0);
  }
  EXPECT(valid > 500);
  if (g_fail) return 1;
  std::puts("host checks ok");
  return 0;
}
