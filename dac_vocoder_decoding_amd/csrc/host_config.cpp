// host_config.cpp -- host-only parts of libvocoder (see host_config.h): no
// HIP calls, compiled into the library and, by the sanitizer test, with g++
// under ASan and UBSan.
#include "host_config.h"

#include <algorithm>
#include <cmath>
#include <cstring>

#define VOC_API extern "C" __attribute__((visibility("default")))

namespace voc {

int total_stride(const voc_config& c) {
  int64_t h = 1;
  for (int b = 0; b < c.n_blocks; ++b) h *= c.stride[b];
  return static_cast<int>(h);
}

voc_status validate(const voc_config* c, std::string* why) {
  auto bad = [&](const char* m) { if (why) *why = m; return VOC_INVALID_PARAMS; };
  if (!c) return bad("config is NULL");
  if (c->abi_version != VOC_ABI_VERSION) return bad("abi_version mismatch");
  if (c->n_blocks < 1 || c->n_blocks > VOC_MAX_BLOCKS) return bad("n_blocks out of range");
  if (c->n_res < 1 || c->n_res > VOC_MAX_RES) return bad("n_res out of range");
  if (c->in_kernel != 7 || c->res_kernel != 7 || c->out_kernel != 7)
    return bad("only kernel size 7 is supported for conv_in, conv1 and conv_out");
  if (c->act != VOC_SNAKE && c->act != VOC_SNAKE_BETA) return bad("unknown act");
  if (c->dtype != VOC_F32 && c->dtype != VOC_BF16) return bad("unknown dtype");
  if (c->snake_log_params != 0 && c->snake_log_params != 1) return bad("snake_log_params must be 0 or 1");
  if (c->convt_crop != 0 && !(c->convt_crop == 1 && c->causal == 1))
    return bad("convt_crop must be 0, or 1 together with causal = 1");
  if (c->tile_frames < 0) return bad("tile_frames must be >= 0");
  const int q = c->dtype == VOC_F32 ? 16 : 32;
  if (c->latent_channels <= 0 || c->latent_channels % q || c->latent_channels > 8192)
    return bad("latent_channels must be a positive multiple of 16 (F32) / 32 (BF16), at most 8192");
  if (c->in_proj < 0 || c->in_proj % q || c->in_proj > 8192)
    return bad("in_proj must be 0 or a positive multiple of 16 (F32) / 32 (BF16), at most 8192");
  if (c->causal != 0 && c->causal != 1) return bad("causal must be 0 or 1");
  if (c->enc_width[0] != 0) {
    for (int b = 0; b <= c->n_blocks; ++b)
      if (c->enc_width[b] <= 0 || c->enc_width[b] % q || c->enc_width[b] > 8192)
        return bad("encoder widths must be positive multiples of 16 (F32) / 32 (BF16), at most 8192");
    for (int b = 0; b < c->n_blocks; ++b)
      if (c->stride[b] % 2) return bad("an encoder needs even strides (pad s/2)");
    if (c->causal) return bad("the encoder is not causal");
  }
  if (c->af_snake != 0 && c->af_snake != 1) return bad("af_snake must be 0 or 1");
  if (c->af_snake && c->causal) return bad("the alias-free Snake is built for non-causal decoders");
  if (c->af_snake && c->enc_width[0] != 0) return bad("the alias-free Snake is built for the decoder only");
  if (c->out_channels != 1 && c->out_channels != 2) return bad("out_channels must be 1 or 2");
  if (c->operand_terms < 0 || c->operand_terms > 2) return bad("operand_terms must be 0, 1 or 2");
  if (c->operand_terms == 2 && (c->dtype != VOC_BF16 || c->af_snake || c->in_proj || c->enc_width[0] != 0))
    return bad("operand_terms = 2 needs a bf16 decoder without the alias-free Snake, dec_in_proj or an encoder");
  for (int b = 0; b <= c->n_blocks; ++b)
    if (c->width[b] <= 0 || c->width[b] % q || c->width[b] > 8192)
      return bad("widths must be positive multiples of 16 (F32) / 32 (BF16), at most 8192");
  if (c->width[c->n_blocks] > 512) return bad("the last width must be at most 512");
  int64_t hop = 1;
  for (int b = 0; b < c->n_blocks; ++b) {
    if (c->stride[b] < 1 || c->stride[b] > 64) return bad("strides must be in [1, 64]");
    hop *= c->stride[b];
    if (hop > (1 << 20)) return bad("hop too large");
  }
  for (int r = 0; r < c->n_res; ++r)
    if (c->dilation[r] < 1 || c->dilation[r] > 9) return bad("dilations must be in [1, 9]");
  return VOC_OK;
}

int64_t floordiv(int64_t a, int64_t b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }

// Smallest halos (H_left, H_right) such that, for every output sample of
// latent frame F, the dependency interval at the input of every layer lies
// inside the frames the tile [F - H_left, F + 1 + H_right) holds at that
// layer's rate.  Intervals are propagated backwards: a k=7 conv at dilation d
// widens them by 3d each side ("same"), or by 6d on the left only (causal);
// ConvTranspose1d (stride s, k = 2s, left crop p = ceil(s/2), or 0 when
// causal) maps outputs [lo, hi] to inputs [ceil((lo + p - 2s + 1)/s),
// floor((hi + p)/s)].  An alias-free Snake widens them by 5 frames each side
// at its rate.  The two ends propagate independently.
void compute_halos(const voc_config& c, int* h_left, int* h_right) {
  const int64_t hop = total_stride(c);
  const int64_t F = 4096;
  const bool causal = c.causal != 0;
  const int64_t kl = causal ? 6 : 3, kr = causal ? 0 : 3;  // k=7 conv reach per unit dilation
  const int64_t af = c.af_snake ? 5 : 0;                   // alias-free Snake reach
  std::vector<int64_t> rate(c.n_blocks + 1);
  rate[0] = 1;
  for (int b = 0; b < c.n_blocks; ++b) rate[b + 1] = rate[b] * c.stride[b];
  *h_left = *h_right = -1;
  for (int H = 0; H < 4096 && (*h_left < 0 || *h_right < 0); ++H) {
    bool ok_l = true, ok_r = true;
    for (int64_t ph = 0; ph < hop; ++ph) {
      int64_t lo = F * hop + ph, hi = lo;
      auto check = [&](int64_t R) {
        ok_l = ok_l && lo >= (F - H) * R;
        ok_r = ok_r && hi < (F + 1 + H) * R;
      };
      lo -= kl + af, hi += kr + af;  // head conv k=7, snake_out
      check(rate[c.n_blocks]);
      for (int b = c.n_blocks - 1; b >= 0; --b) {
        for (int r = c.n_res - 1; r >= 0; --r) {  // Snake2, conv1, Snake1 (conv2 is k=1)
          lo -= kl * c.dilation[r] + 2 * af, hi += kr * c.dilation[r] + 2 * af;
          check(rate[b + 1]);
        }
        const int64_t s = c.stride[b], p = causal ? 0 : (s + 1) / 2;
        lo = -floordiv(-(lo + p - 2 * s + 1), s);
        hi = floordiv(hi + p, s);
        lo -= af, hi += af;  // the block's Snake
        check(rate[b]);
      }
      lo -= kl, hi += kr;  // conv_in
      check(1);
    }
    if (ok_l && *h_left < 0) *h_left = H;
    if (ok_r && *h_right < 0) *h_right = H;
  }
}

int compute_halo(const voc_config& c) {
  int hl, hr;
  compute_halos(c, &hl, &hr);
  return hl < 0 || hr < 0 ? -1 : std::max(hl, hr);
}

// The GEMM stages activation tiles through buffer loads with 32-bit byte
// offsets into one 64-byte-row channel plane.  A launch is addressable when
// its plane (frames, the lb context frames before it, and the 512 * S rows
// a tile may read past its end, S the input stride) stays below 2^32 bytes
// with a 64 KB guard, so that the offsets of rows before the plane (tiles at
// the left edge) wrap to values past its end and read as zero.
const int64_t kPlaneLimitBytes = (int64_t(1) << 32) - (int64_t(1) << 16);
const int64_t kStreamCtxMax = 54;  // the longest carried context: 6 * dilation 9

bool gemm_plane_ok(int64_t plane_frames, int64_t lb, int64_t S) {
  return plane_frames >= 0 && (plane_frames + lb + 512 * S) * kChunkBytes <= kPlaneLimitBytes;
}

// Largest GEMM input rate (frames per latent frame) of the decoder stack:
// the ConvTranspose1d of block b reads frames at rate_b, and the residual
// convs of block b run as GEMMs at rate_{b+1} unless the unit is fused
// (the fused unit addresses h with 64-bit pointers).  Alias-free (and
// split-Snake) stacks run every unit as a GEMM pair.
int64_t gemm_rate_max(const voc_config& g, int op, bool units_unfused) {
  int64_t rate = 1, mx = 1;
  for (int b = 0; b < g.n_blocks; ++b) {
    mx = std::max(mx, rate);
    rate *= g.stride[b];
    const bool fused = !units_unfused && res_unit_tile(op, g.width[b + 1], false) > 0;
    if (!fused) mx = std::max(mx, rate);
  }
  return mx;
}

// Largest latent frames per decoded row (a whole row, or a tile with its
// halos) whose GEMM planes are all addressable (streams' context included).
int64_t max_row_frames(const voc_config& g, int op, bool units_unfused) {
  const int64_t per = gemm_rate_max(g, op, units_unfused);
  const int64_t frames = kPlaneLimitBytes / kChunkBytes - kStreamCtxMax - 512;
  return frames / per;
}


// ----------------------------------------------------------- weight names

std::vector<int64_t> squeeze(const int64_t* shape, int nd) {
  std::vector<int64_t> v;
  for (int i = 0; i < nd; ++i)
    if (shape[i] != 1) v.push_back(shape[i]);
  return v;
}

std::map<std::string, Expect> expected_tensors(const voc_config& g) {
  std::map<std::string, Expect> m;
  auto sq = [](std::vector<int64_t> v) {
    std::vector<int64_t> r;
    for (auto x : v)
      if (x != 1) r.push_back(x);
    return r;
  };
  auto conv = [&](const std::string& p, int64_t d0, int64_t d1, int64_t k, int64_t nbias) {
    m[p + ".weight_v"] = {sq({d0, d1, k})};
    m[p + ".weight_g"] = {sq({d0})};
    m[p + ".bias"] = {sq({nbias})};
  };
  auto snake = [&](const std::string& p, int64_t ch) {
    m[p + ".alpha"] = {sq({ch})};
    if (g.act == VOC_SNAKE_BETA) m[p + ".beta"] = {sq({ch})};
  };
  if (g.in_proj > 0) {  // plain Conv1d k=1, no weight norm
    m["dec_in_proj.weight"] = {sq({g.in_proj, g.latent_channels, 1})};
    m["dec_in_proj.bias"] = {sq({g.in_proj})};
  }
  conv("conv_in", g.width[0], g.in_proj > 0 ? g.in_proj : g.latent_channels, 7, g.width[0]);
  for (int b = 0; b < g.n_blocks; ++b) {
    const std::string p = "blocks." + std::to_string(b);
    const int cin = g.width[b], cout = g.width[b + 1];
    snake(p + ".snake1", cin);
    conv(p + ".conv_t1", cin, cout, 2 * g.stride[b], cout);
    for (int r = 0; r < g.n_res; ++r) {
      const std::string q = p + ".res_units." + std::to_string(r);
      snake(q + ".snake1", cout);
      conv(q + ".conv1", cout, cout, 7, cout);
      snake(q + ".snake2", cout);
      conv(q + ".conv2", cout, cout, 1, cout);
    }
  }
  snake("snake_out", g.width[g.n_blocks]);
  conv("conv_out", g.out_channels, g.width[g.n_blocks], 7, g.out_channels);
  if (g.enc_width[0] > 0) {  // the encoder: decoder strides in reverse order
    const int* E = g.enc_width;
    conv("encoder.conv_in", E[0], 1, 7, E[0]);
    for (int b = 0; b < g.n_blocks; ++b) {
      const std::string q = "encoder.blocks." + std::to_string(b);
      for (int r = 0; r < g.n_res; ++r) {
        const std::string u = q + ".res_units." + std::to_string(r);
        snake(u + ".snake1", E[b]);
        conv(u + ".conv1", E[b], E[b], 7, E[b]);
        snake(u + ".snake2", E[b]);
        conv(u + ".conv2", E[b], E[b], 1, E[b]);
      }
      snake(q + ".snake", E[b]);
      conv(q + ".down", E[b + 1], E[b], 2 * g.stride[g.n_blocks - 1 - b], E[b + 1]);
    }
    snake("encoder.snake_out", E[g.n_blocks]);
    conv("encoder.conv_out", E[g.n_blocks], E[g.n_blocks], 3, E[g.n_blocks]);
    conv("encoder.proj", g.latent_channels, E[g.n_blocks], 1, g.latent_channels);
  }
  return m;
}

bool all_finite(const float* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!std::isfinite(p[i])) return false;
  return true;
}

int64_t numel(const voc_tensor& t) {
  int64_t n = 1;
  for (int i = 0; i < t.ndim; ++i) n *= t.shape[i];
  return n;
}


// Kept latent frames [lo, hi) of window k of n (window stitching): every
// window but the first drops crop_left frames on the left, every window but
// the last drops crop_right on the right.
void window_keep(int64_t k, int64_t n, int64_t L, int64_t L_last, int64_t cl, int64_t cr, int64_t* lo,
                 int64_t* hi) {
  const int64_t len = k == n - 1 ? L_last : L;
  *lo = k > 0 ? cl : 0;
  *hi = len - (k < n - 1 ? cr : 0);
}

bool windows_valid(int64_t n, int64_t L, int64_t L_last, int64_t cl, int64_t cr) {
  if (n <= 0 || L <= 0 || L_last <= 0 || L_last > L || cl < 0 || cr < 0) return false;
  // The first window, a middle one (they are all alike) and the last must
  // each keep at least one frame.
  const int64_t ks[3] = {0, n > 2 ? 1 : 0, n - 1};
  for (int64_t k : ks) {
    int64_t lo, hi;
    window_keep(k, n, L, L_last, cl, cr, &lo, &hi);
    if (hi <= lo) return false;
  }
  return true;
}

// Modified Bessel function of the first kind, order 0, from its power series
// I0(x) = sum_k ((x/2)^k / k!)^2 (all terms positive; converges fast for the
// arguments of a Kaiser window).
double bessel_i0(double x) {
  double term = 1.0, sum = 1.0;
  for (int k = 1; k < 64; ++k) {
    term *= (x / (2.0 * k)) * (x / (2.0 * k));
    sum += term;
    if (term < 1e-17 * sum) break;
  }
  return sum;
}

// The alias-free Snake's low-pass (a windowed-sinc design, Kaiser's window,
// as the BigVGAN anti-aliased activation uses it): 12 taps, cutoff 0.25
// cycles per sample of the 2x rate (the original Nyquist frequency),
// transition half-width 0.3; Kaiser's empirical formulas give the window
// parameter beta from the attenuation
// A = 2.285 (taps/2 - 1) pi (4 * half-width) + 7.95 dB; the taps sit at
// half-integer times -5.5 .. 5.5 and are normalised to unit sum.  fe and fo
// are the polyphase taps of the upsampler (gain 2): output sample 2m uses
// 2 f[11 - 2k] on x[m - 3 + k], sample 2m+1 uses 2 f[10 - 2k] on x[m - 2 + k].
void design_af_filter(float* fe, float* fo, float* fd) {
  const int K = kAfTaps, half = K / 2;
  const double cutoff = 0.25, half_width = 0.3;
  const double A = 2.285 * (half - 1) * M_PI * (4.0 * half_width) + 7.95;
  const double beta = A > 50.0 ? 0.1102 * (A - 8.7)
                      : A >= 21.0 ? 0.5842 * std::pow(A - 21.0, 0.4) + 0.07886 * (A - 21.0)
                                  : 0.0;
  double f[kAfTaps], sum = 0.0;
  for (int n = 0; n < K; ++n) {
    const double r = 2.0 * n / (K - 1) - 1.0;
    const double w = bessel_i0(beta * std::sqrt(std::max(0.0, 1.0 - r * r))) / bessel_i0(beta);
    const double t = 2.0 * cutoff * (n - half + 0.5);
    const double sinc = std::sin(M_PI * t) / (M_PI * t);  // t is never 0 (half-integer times)
    f[n] = 2.0 * cutoff * w * sinc;
    sum += f[n];
  }
  for (int n = 0; n < K; ++n) fd[n] = static_cast<float>(f[n] / sum);
  for (int k = 0; k < 6; ++k) {
    fe[k] = static_cast<float>(2.0 * f[11 - 2 * k] / sum);
    fo[k] = static_cast<float>(2.0 * f[10 - 2 * k] / sum);
  }
}
}  // namespace voc

using namespace voc;

// ============================================================ host-only ABI

VOC_API void voc_config_default(voc_config* cfg) {
  if (!cfg) return;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->abi_version = VOC_ABI_VERSION;
  cfg->latent_channels = 64;
  cfg->n_blocks = 4;
  const int w[5] = {1024, 512, 256, 128, 64};
  const int st[4] = {8, 8, 4, 2};
  for (int i = 0; i < 5; ++i) cfg->width[i] = w[i];
  for (int i = 0; i < 4; ++i) cfg->stride[i] = st[i];
  cfg->in_kernel = cfg->res_kernel = cfg->out_kernel = 7;
  cfg->n_res = 3;
  cfg->dilation[0] = 1;
  cfg->dilation[1] = 3;
  cfg->dilation[2] = 9;
  cfg->act = VOC_SNAKE;
  cfg->dtype = VOC_F32;
  cfg->out_channels = 1;
}

VOC_API voc_status voc_config_validate(const voc_config* cfg) { return validate(cfg, nullptr); }

VOC_API int64_t voc_config_hop(const voc_config* cfg) {
  if (validate(cfg, nullptr) != VOC_OK) return VOC_INVALID_PARAMS;
  return total_stride(*cfg);
}

VOC_API int voc_config_halo(const voc_config* cfg) {
  if (validate(cfg, nullptr) != VOC_OK) return VOC_INVALID_PARAMS;
  return compute_halo(*cfg);
}

VOC_API int64_t voc_config_max_frames(const voc_config* cfg) {
  if (validate(cfg, nullptr) != VOC_OK) return VOC_INVALID_PARAMS;
  return max_row_frames(*cfg, cfg->dtype == VOC_F32 ? OP_F32 : OP_BF16, cfg->af_snake != 0);
}
