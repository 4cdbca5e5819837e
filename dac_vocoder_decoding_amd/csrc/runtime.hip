// runtime.hip -- host side of libvocoder: the C ABI declared in vocoder.h.
//
// Validation, the exact tiling halos, weight ingestion (device-side fold and
// repack), the alias-free Snake's low-pass design, workspace management, the
// launch sequences of a decode (plain or alias-free), a windowed decode, a
// stream chunk (with the per-layer carried context) and an encode,
// per-launch profiling and the debug stage runner.  No exception crosses the
// ABI.
#include "../../include/vocoder.h"
#include "internal.h"

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#define VOC_API extern "C" __attribute__((visibility("default")))

using namespace voc;

namespace {

std::string g_create_error;

// The no-allocation decode's workspace (vocoder_decode_noalloc): a fixed
// device array, one copy per GPU, held until the process ends.  Host code
// never passes this name to a kernel or a copy: the address of each
// device's copy comes from hipGetSymbolAddress, taken once per device at
// vocoder_create with that device current.
constexpr size_t kScratchBytes = VOC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

struct SnakeDev {
  float* alpha = nullptr;   // alpha / pi per channel
  float* invden = nullptr;  // 1 / (2 (den + 1e-9)) per channel
};
struct ConvDev {
  void* w = nullptr;
  float* bias = nullptr;
  int cin = 0, cout = 0, taps = 0, dil = 1, ups = 1, crop = 0, M = 0;
  int causal = 0;  // k=7: left padding (K-1)*d instead of "same"
  int down = 1;    // > 1: strided conv (k = 2*down, stride down, pad down/2) as 2 taps
  int terms = 1;   // 2: its input is a two-term operand (2 * cin channels; w holds every
                   // input chunk plane twice)
};
struct UnitDev {
  SnakeDev a1, a2;
  ConvDev c1, c2;
};
struct BlockDev {
  SnakeDev act;
  ConvDev ct;
  std::vector<UnitDev> units;
};
struct EncBlockDev {
  std::vector<UnitDev> units;
  SnakeDev act;     // Snake ahead of the strided conv
  ConvDev down;
};
struct EncoderDev {
  ConvDev conv_in;  // 1 input channel, packed as one zero-padded chunk
  std::vector<EncBlockDev> blocks;
  SnakeDev out_act;
  ConvDev conv_out, proj;
};
struct Weights {
  EncoderDev enc;   // (enc.conv_in.cout == 0: no encoder)
  ConvDev in_proj;  // dec_in_proj (cout == 0: none)
  ConvDev conv_in;
  std::vector<BlockDev> blocks;
  SnakeDev head_act;
  float* head_w = nullptr;
  float head_bias[2] = {0.f, 0.f};
  std::vector<void*> allocs;
};

struct ProfRec {
  int kind;
  double flops, bytes;
  hipEvent_t e0, e1;
};

}  // namespace

struct voc_ctx {
  voc_config cfg{};
  int device = 0;
  int op = OP_F32;
  int64_t hop = 1;
  int halo_l = 0, halo_r = 0;  // receptive-field halos in latent frames (left, right)
  // Alias-free Snake low-pass (af_snake): polyphase upsampling taps and the
  // downsampling taps, fp32 (see design_af_filter).
  float af_fe[6] = {}, af_fo[6] = {}, af_fd[kAfTaps] = {};
  std::string err;
  bool loaded = false;
  Weights W;
  // workspace
  void* ws = nullptr;
  size_t ws_bytes = 0;
  size_t ws_cap = 0;
  // profiling
  bool prof = false;
  uint32_t prof_kinds = 0;  // kinds timed with events (0 = all)
  std::vector<ProfRec> pending;
  std::vector<hipEvent_t> free_events;
  voc_profile_stat stats[VOC_K_COUNT]{};
  // cached row metadata of the last decode
  std::vector<int64_t> rows_key;  // what the uploaded metadata describes (empty: nothing)
  int force_variant[VOC_K_COUNT] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1, -1};  // ablation overrides
  bool no_fuse = false;                 // ablation: always run conv1 and conv2 apart
  int m_order = -1;                     // ablation: conv tile order (-1 auto, 0 N fastest, 1 M fastest)
  int ru_xh = 1;                        // fused units compute Snake1 from h (0: read an operand tensor)
  int terms = 1;                        // matrix-core operand terms (voc_config::operand_terms)
  bool split_snake = false;             // ablation: every plain Snake as a launch of its own
  bool split_tanh = false;              // ablation: tanh as a pass of its own after the head
  bool head_no_tanh = false;            // set during a split-tanh decode
  bool col2im = false;                  // ablation: ConvTranspose1d as GEMM + col2im
  float* col_buf = nullptr;             // its column matrix (and a zero bias), grown on demand
  size_t col_bytes = 0;
  float* col_zero = nullptr;
  // streaming (causal configurations): the carried context of every layer
  // with one ([planes][ctx][64 bytes], two copies that alternate by chunk),
  // in the order conv_in, per block: ConvTranspose1d then its units, head.
  struct LayerState {
    int ctx = 0;                  // frames of context
    int64_t planes_per_row = 0;   // frame-row planes of the layer's input
    int row_bytes = kChunkBytes;  // bytes per frame row (operand 64; residual 16 elements)
    size_t off[2] = {0, 0};       // byte offsets of the two copies in st_mem
  };
  std::vector<LayerState> st_layers;
  void* st_mem = nullptr;
  size_t st_mem_bytes = 0;
  int64_t st_rows = 0;          // streams since the last reset (0: none)
  int st_par = 0;               // which copy holds the current context
  int st_margin = 0;            // margin frames in front of every activation plane
  bool st_active = false;       // the stack runs a stream chunk (exchanges on)
  int mg = 0;                   // margin frames of the activation planes being decoded
  std::vector<int64_t> meta_dst;  // host copies kept alive for async uploads
  std::vector<int> meta_int;
  // the no-allocation decode: this device's copy of the scratch array, and
  // while such a call runs the workspace it substitutes for ws
  void* scratch = nullptr;
  void* ws_override = nullptr;
  size_t ws_override_bytes = 0;
  // cancellation hook (vocoder_set_cancel): polled before a call enqueues
  // work and between groups of cancel_group units
  int64_t frames_cap = 0;        // test switch: a lower row-frame limit (0: none)
  voc_cancel_fn cancel_fn = nullptr;
  void* cancel_user = nullptr;
  int64_t cancel_group = 1;
};

namespace {

voc_status fail(voc_ctx* c, voc_status st, const std::string& msg) {
  if (c) c->err = msg; else g_create_error = msg;
  return st;
}

voc_status hip_fail(voc_ctx* c, hipError_t e, const char* what) {
  std::string m = std::string(what) + ": " + hipGetErrorString(e);
  return fail(c, e == hipErrorOutOfMemory ? VOC_OOM : VOC_DEVICE_ERROR, m);
}

// ------------------------------------------------------------- profiling
hipEvent_t take_event(voc_ctx* c) {
  if (!c->free_events.empty()) {
    hipEvent_t e = c->free_events.back();
    c->free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

voc_status finalize_profile(voc_ctx* c) {
  for (auto& r : c->pending) {
    float ms = 0.f;
    if (r.e0) {  // a timed launch
      hipError_t e = hipEventSynchronize(r.e1);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.e0, r.e1);
      if (e != hipSuccess) return hip_fail(c, e, "profile event");
      c->free_events.push_back(r.e0);
      c->free_events.push_back(r.e1);
    }
    auto& st = c->stats[r.kind];
    st.launches += 1;
    st.ms += ms;
    st.flops += r.flops;
    st.bytes += r.bytes;
  }
  c->pending.clear();
  return VOC_OK;
}

// Launch wrapper: records events around the launch when profiling is on.
template <class F>
voc_status launch(voc_ctx* c, hipStream_t s, int kind, double flops, double bytes, const char* what,
                  F&& fn) {
  ProfRec rec{kind, flops, bytes, nullptr, nullptr};
  const bool timed = c->prof && (c->prof_kinds == 0 || ((c->prof_kinds >> kind) & 1u));
  if (timed) {
    rec.e0 = take_event(c);
    rec.e1 = take_event(c);
    if (!rec.e0 || !rec.e1) return fail(c, VOC_DEVICE_ERROR, "hipEventCreate failed");
    (void)hipEventRecord(rec.e0, s);
  }
  hipError_t e = fn();
  if (e != hipSuccess) return hip_fail(c, e, what);
  if (timed) (void)hipEventRecord(rec.e1, s);
  if (c->prof) c->pending.push_back(rec);
  return VOC_OK;
}

// ------------------------------------------------------------- workspace
struct Plan {
  int rows, T;            // rows and latent frames per row
  int mg;                 // margin frames in front of every activation plane (streams)
  size_t off_xlat, off_h, off_h2, off_s0, off_s1, off_u, off_meta, bytes;
};

size_t align_up(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Whether the residual units of width C run fused with their conv1 operand
// computed from h in the kernel (Snake1 at staging): their producers then
// write no operand tensor, and h alternates between two buffers.  Every
// fused width does (per-layer kernel traces on MI355X: the ConvTranspose1d
// feeding such a block saves 15-23 % and the first two units 2-14 %, while
// the last unit of a block is 3-9 % slower; the mono codec's 96-channel
// block as a whole 3.5 % faster).
bool unit_xh(const voc_ctx* c, int C) {
  return !c->cfg.af_snake && !c->split_snake && c->ru_xh && !c->no_fuse && res_unit_tile(c->op, C, false, c->terms) > 0;
}

// Largest latent frames per decoded row this context's decoder can address
// (its GEMM planes below 4 GiB; the ablation switches move units onto GEMMs).
int64_t row_frames_limit(const voc_ctx* c) {
  const int64_t m = max_row_frames(c->cfg, c->op, c->cfg.af_snake || c->split_snake || c->no_fuse);
  return c->frames_cap > 0 ? std::min(m, c->frames_cap) : m;
}

bool any_unit_xh(const voc_ctx* c) {
  for (int b = 0; b < c->cfg.n_blocks; ++b)
    if (unit_xh(c, c->cfg.width[b + 1])) return true;
  return false;
}

// The head's Snake_out, when the head applies it while loading the fp16
// residual stream (bf16 decoders without standalone Snake launches); null
// when the last producer stores Snake_out(h) in fp32 for it.
const SnakeDev* head_snake_at_load(const voc_ctx* c) {
  return c->op == OP_BF16 && c->terms == 1 && !c->cfg.af_snake && !c->split_snake ? &c->W.head_act : nullptr;
}

// Bytes per residual-stream element: fp32, or fp16 for one-term bf16 decoders
// (two-term decoders keep h in fp32, whose precision their operands need).
int hsz(const voc_ctx* c) { return c->terms == 2 ? 4 : h_size(c->op); }

Plan make_plan(const voc_ctx* c, int rows, int T, int mg = 0) {
  const voc_config& g = c->cfg;
  const size_t es = op_size(c->op);
  size_t max_act = 0;
  int64_t t = T;
  max_act = std::max<size_t>(max_act, static_cast<size_t>(g.width[0]) * (t + mg));
  max_act = std::max<size_t>(max_act, static_cast<size_t>(g.in_proj) * (t + mg));  // dec_in_proj out (in u)
  for (int b = 0; b < g.n_blocks; ++b) {
    t *= g.stride[b];
    max_act = std::max<size_t>(max_act, static_cast<size_t>(g.width[b + 1]) * (t + mg));
  }
  Plan p{};
  p.rows = rows;
  p.T = T;
  p.mg = mg;
  size_t o = 0;
  p.off_xlat = o; o = align_up(o + es * rows * static_cast<size_t>(g.latent_channels) * (T + mg));
  // The residual-stream buffers are sized for fp32 elements: the last one
  // holds the head's input, Snake_out(h), in fp32 also for bf16 decoders.
  p.off_h = o;    o = align_up(o + 4 * rows * max_act);
  p.off_h2 = o;   if (any_unit_xh(c) || g.af_snake || c->split_snake) o = align_up(o + 4 * rows * max_act);
  // Operand tensors hold c->terms bf16 terms per element (two-term operands).
  const size_t eo = es * c->terms;
  p.off_s0 = o;   o = align_up(o + eo * rows * max_act);
  p.off_s1 = o;   o = align_up(o + eo * rows * max_act);
  p.off_u = o;    o = align_up(o + eo * rows * max_act);
  p.off_meta = o; o = align_up(o + static_cast<size_t>(rows) * (5 * sizeof(int) + sizeof(int64_t)) + 64);
  p.bytes = o;
  return p;
}

// The encoder's workspace: the audio as a one-chunk operand, then the same
// activation buffers as a decode, sized for the encoder's widths and rates.
Plan make_enc_plan(const voc_ctx* c, int rows, int T) {
  const voc_config& g = c->cfg;
  const size_t es = op_size(c->op);
  int64_t t = T * c->hop;
  size_t max_act = static_cast<size_t>(g.latent_channels) * T;
  bool xh = false;
  for (int b = 0; b <= g.n_blocks; ++b) {
    max_act = std::max<size_t>(max_act, static_cast<size_t>(g.enc_width[b]) * t);
    if (b < g.n_blocks) {
      xh = xh || unit_xh(c, g.enc_width[b]);
      t /= g.stride[g.n_blocks - 1 - b];
    }
  }
  Plan p{};
  p.rows = rows;
  p.T = T;
  size_t o = 0;
  p.off_xlat = o; o = align_up(o + static_cast<size_t>(rows) * T * c->hop * kChunkBytes);
  p.off_h = o;    o = align_up(o + 4 * rows * max_act);
  p.off_h2 = o;   if (xh) o = align_up(o + 4 * rows * max_act);
  p.off_s0 = o;   o = align_up(o + es * rows * max_act);
  p.off_s1 = o;   o = align_up(o + es * rows * max_act);
  p.off_u = o;    o = align_up(o + es * rows * max_act);
  p.off_meta = o; o = align_up(o + static_cast<size_t>(rows) * (5 * sizeof(int) + sizeof(int64_t)) + 64);
  p.bytes = o;
  return p;
}

// The workspace base: the library-owned allocation, or the scratch array
// during a no-allocation decode.
char* ws_base(const voc_ctx* c) { return static_cast<char*>(c->ws_override ? c->ws_override : c->ws); }

voc_status ensure_ws(voc_ctx* c, size_t bytes) {
  if (c->ws_override) {  // never allocates: the caller has sized the rows to fit
    if (bytes <= c->ws_override_bytes) return VOC_OK;
    return fail(c, VOC_INVALID_PARAMS, "workspace of " + std::to_string(bytes) +
                                           " bytes exceeds the no-allocation scratch");
  }
  if (bytes <= c->ws_bytes) return VOC_OK;
  if (c->ws_cap && bytes > c->ws_cap)
    return fail(c, VOC_OOM, "workspace of " + std::to_string(bytes) +
                                " bytes exceeds VOC_MAX_WORKSPACE_BYTES");
  if (c->ws) {
    (void)hipDeviceSynchronize();
    (void)hipFree(c->ws);
    c->ws = nullptr;
    c->ws_bytes = 0;
  }
  c->rows_key.clear();  // row metadata lived in the old workspace
  hipError_t e = hipMalloc(&c->ws, bytes);
  if (e != hipSuccess) {
    c->ws = nullptr;
    return hip_fail(c, e, "workspace hipMalloc");
  }
  c->ws_bytes = bytes;
  return VOC_OK;
}

struct Bufs {
  void* xlat;
  float* h;
  float* h2;  // second residual-stream buffer (units with the operand from h)
  void* s[2];
  void* u;
  RowInfo rows;
};

Bufs bufs(voc_ctx* c, const Plan& p) {
  char* b = ws_base(c);
  Bufs r{};
  // Activation pointers address frame 0 of the first plane; with a margin
  // every plane starts mg frames (64-byte rows) earlier.
  const size_t mgb = static_cast<size_t>(p.mg) * kChunkBytes;
  r.xlat = b + p.off_xlat + mgb;
  // (The residual-stream buffers keep fp32-sized margins: fp16 planes use
  // half of each margin, the head's fp32 input all of it.)
  r.h = reinterpret_cast<float*>(b + p.off_h + mgb);
  r.h2 = reinterpret_cast<float*>(b + p.off_h2 + mgb);
  r.s[0] = b + p.off_s0 + mgb;
  r.s[1] = b + p.off_s1 + mgb;
  r.u = b + p.off_u + mgb;
  char* m = b + p.off_meta;
  r.rows.dst = reinterpret_cast<const int64_t*>(m);
  const int* ib = reinterpret_cast<const int*>(m + sizeof(int64_t) * p.rows);
  r.rows.len = ib;
  r.rows.src_b = ib + p.rows;
  r.rows.start = ib + 2 * p.rows;
  r.rows.keep_lo = ib + 3 * p.rows;
  r.rows.keep_hi = ib + 4 * p.rows;
  return r;
}

// Upload row metadata: rows = B * tiles; per row its window of the latent.
// The host vectors are kept in the context until the next upload, so the
// asynchronous copy never reads freed memory.
voc_status upload_rows(voc_ctx* c, const Plan& p, std::vector<int64_t>&& dst_in,
                       std::vector<int>&& ints_in, hipStream_t s) {
  c->meta_dst = std::move(dst_in);
  c->meta_int = std::move(ints_in);
  const std::vector<int64_t>& dst = c->meta_dst;
  const std::vector<int>& ints = c->meta_int;
  char* m = ws_base(c) + p.off_meta;
  hipError_t e = hipMemcpyAsync(m, dst.data(), dst.size() * sizeof(int64_t), hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(m + sizeof(int64_t) * p.rows, ints.data(), ints.size() * sizeof(int),
                       hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return hip_fail(c, e, "row metadata upload");
  return VOC_OK;
}

// ------------------------------------------------------------ conv launch
// Tile choice: padding efficiency of M and N x wave quantization over two
// workgroups per CU x a relative speed of the tile family for the operand
// dtype and tap count, measured on MI355X (a sweep forcing each family on
// the full-window fp32 and batched-window bf16 decodes).  The narrow fp32
// tiles: for 7 taps the 32-row tile (26 KB of LDS per stage, three
// workgroups per CU against two for the 64-row tile) is 1-3 % faster on
// every k=7 layer of the fp32 workloads and 23 % faster where one row of
// 3000 frames leaves the 64-row tiles short of workgroups; the 16-row tile
// serves 16-channel units (23 us against 67 us for a 64-row tile three
// quarters empty).  For 1 and 2 taps the narrow tiles measured level with
// the 64-row ones and are taken when they fill the chip better.  The bf16
// 1-tap 64x128 tile runs 0.88-0.94 of the 128x128 one's rate on the wide
// units, also where the 128x128 grid leaves its last round half empty
// (512 channels x 5.5 k frames x 16 rows: 113 against 128 us).
int pick_variant(int op, int taps, int M, int N, int rows) {
  //                                  128x256 64x256 96x256 128x128 64x128 192x128 16x128 32x128
  static const double f32[CV_COUNT]   = {0.60, 0.90, 0.85, 0.90, 1.00, 0.70, 0.50, 0.90};
  static const double f32_t7[CV_COUNT] = {0.00, 0.90, 0.85, 0.00, 1.00, 0.00, 0.00, 1.05};
  static const double bf_t2[CV_COUNT] = {0.90, 0.80, 0.85, 1.00, 0.75, 0.92, 0.00, 0.00};
  static const double bf_t7[CV_COUNT] = {0.00, 1.00, 1.00, 0.00, 0.88, 0.00, 0.00, 0.00};
  static const double bf_t1[CV_COUNT] = {0.46, 0.94, 0.80, 1.00, 0.88, 0.68, 0.00, 0.00};
  const double* speed = op == OP_F32 ? (taps == 7 ? f32_t7 : f32)
                                     : taps == 2 ? bf_t2 : taps == 7 ? bf_t7 : bf_t1;
  // The 16-row 7-tap tile exactly when M <= 16 (the other families would
  // leave at least three quarters of their rows empty).
  if (taps == 7 && op == OP_F32 && M <= 16) return CV_16x128;
  int best = CV_64x128;
  double best_score = -1.0;
  for (int v = 0; v < CV_COUNT; ++v) {
    if (!conv_variant_ok(v, taps)) continue;
    if (taps == 7 && v == CV_16x128) continue;
    const int bm = conv_variant_bm(v), bn = conv_variant_bn(v);
    const int64_t mt = (M + bm - 1) / bm, nt = (N + bn - 1) / bn;
    const int64_t tiles = mt * nt * rows;
    const double pad = static_cast<double>(M) * N / (static_cast<double>(mt) * bm * nt * bn);
    const int64_t slots = 256 * 2;
    const int64_t waves = (tiles + slots - 1) / slots;
    const double quant = static_cast<double>(tiles) / static_cast<double>(waves * slots);
    const double score = pad * quant * speed[v];
    if (score > best_score) {
      best_score = score;
      best = v;
    }
  }
  return best;
}

struct ConvIO {
  const void* x;
  int T_in;     // allocated frames per row of x
  int rate_in;  // frames per latent frame of x
  float* h_out;
  const float* res;
  void* s_out;
  const SnakeDev* snake_next;  // Snake applied for s_out
  const SnakeDev* h_snake;     // if set, h_out receives Snake(h) (the head's)
};

voc_status run_conv(voc_ctx* c, const ConvDev& L, const ConvIO& io, int rows, const int* row_len,
                    int kind, hipStream_t s) {
  ConvArgs a{};
  a.x = io.x;
  a.T_in = io.T_in + c->mg;  // plane length (margin included)
  a.Cin = L.cin * L.terms;   // a two-term operand: the low terms as further channels
  a.row_len = row_len;
  a.rate_in = io.rate_in;
  a.rate_out = L.down > 1 ? io.rate_in / L.down : io.rate_in * L.ups;
  a.in_stride = L.down;
  a.w = L.w;
  a.M = L.M;
  a.Cout = L.cout;
  if (L.down > 1) {  // strided conv: taps at phase-stream frames n and n+1
    a.off0 = 0;
    a.offstep = 1;
    a.min_off = 0;
    a.halo = 1;
    a.N = io.T_in / L.down;
  } else if (L.taps == 2) {  // polyphase ConvTranspose1d: taps at x[q], x[q-1]
    a.off0 = 0;
    a.offstep = -1;
    a.min_off = -1;
    a.halo = 1;
    a.N = io.T_in + (L.crop > 0 ? 1 : 0);  // a left crop shifts the last outputs to n = T_in
  } else {  // taps at x[n + j*dil - P]: "same" P = (taps-1)/2*dil, causal P = (taps-1)*dil
    const int P = (L.causal ? L.taps - 1 : (L.taps - 1) / 2) * L.dil;
    a.off0 = -P;
    a.offstep = L.dil;
    a.min_off = -P;
    a.halo = (L.taps - 1) * L.dil;
    a.N = io.T_in;
  }
  const int t_out = L.down > 1 ? io.T_in / L.down : io.T_in * L.ups;
  a.T_out = t_out + c->mg;
  a.ups = L.ups;
  a.crop = L.crop;
  // A stream chunk reads its carried context: x[n - 1] for the transposed
  // conv, (K-1)*d frames for a causal k=7 conv.
  a.lb = c->st_active ? (L.taps == 2 ? 1 : -a.min_off) : 0;
  a.bias = L.bias;
  a.h_out = io.h_out;
  a.res = io.res;
  a.s_out = io.s_out;
  a.two_term = c->terms == 2 ? 1 : 0;  // every operand such a decoder writes feeds a two-term input
  a.s_alpha = io.snake_next ? io.snake_next->alpha : nullptr;
  a.s_invden = io.snake_next ? io.snake_next->invden : nullptr;
  a.hs_scale = io.h_snake ? io.h_snake->alpha : nullptr;
  a.hs_h = io.h_snake ? io.h_snake->invden : nullptr;
  a.rows = rows;
  if (!gemm_plane_ok(a.T_in, a.lb, L.down))
    return fail(c, VOC_INVALID_PARAMS,
                "a convolution's input plane exceeds the 4 GiB range of the GEMM's 32-bit buffer offsets "
                "(decode in time tiles)");
  int v = pick_variant(c->op, L.taps, L.M, a.N, rows);
  if (c->force_variant[kind] >= 0 && conv_variant_ok(c->force_variant[kind], L.taps))
    v = c->force_variant[kind];
  a.n_tiles = (a.N + conv_variant_bn(v) - 1) / conv_variant_bn(v);
  a.m_tiles = (a.M + conv_variant_bm(v) - 1) / conv_variant_bm(v);
  // Weights of at most 2 MB stay resident in a 4 MB XCD L2 next to the
  // activation tiles, so the M-tiles of one N-range can run together.
  const double wbytes = static_cast<double>(L.taps) * L.M * L.cin * L.terms * L.down * op_size(c->op);
  a.m_fast = c->m_order >= 0 ? c->m_order : (a.m_tiles > 1 && wbytes <= 2.0 * (1 << 20));
  // Algorithmic work: every input frame meets every tap (direct convolution;
  // a strided conv: every output frame meets its 2s taps).
  const double frames_in = static_cast<double>(rows) * io.T_in;
  const double frames_out = static_cast<double>(rows) * t_out;
  const double flops = L.down > 1 ? 2.0 * frames_out * L.cin * L.cout * 2 * L.down
                                  : 2.0 * frames_in * L.cin * L.cout * (L.taps == 2 ? 2 * L.ups : L.taps);
  const double es = op_size(c->op);
  double bytes = frames_in * L.cin * L.terms * es + wbytes;
  if (io.h_out) bytes += frames_out * L.cout * hsz(c);
  if (io.res) bytes += frames_out * L.cout * hsz(c);
  if (io.s_out) bytes += frames_out * L.cout * es * c->terms;
  const int op = c->op;
  return launch(c, s, kind, flops, bytes, "conv launch",
                [&] {
                  const int tag = kind == VOC_K_CONV_IN || kind == VOC_K_IN_PROJ ? 1 : kind == VOC_K_ENC_OUT ? 3 : 0;
                  return launch_conv(op, L.taps, v, tag, a, s);
                });
}

// A ConvTranspose1d launch: the polyphase GEMM, or in the col2im ablation a
// plain GEMM into the column matrix z[k*Cout + o][n] (the polyphase packing
// read with 2s*Cout rows and one tap is exactly that GEMM's weight) followed
// by the overlap-add, which applies the polyphase GEMM's epilogue.
voc_status run_convt(voc_ctx* c, const ConvDev& L, const ConvIO& io, int rows, const int* row_len,
                     hipStream_t s) {
  if (!c->col2im) return run_conv(c, L, io, rows, row_len, VOC_K_CONVT, s);
  const int mcol = 2 * L.ups * L.cout;
  const size_t need = static_cast<size_t>(rows) * mcol * (io.T_in + c->mg) * sizeof(float);
  if (need > c->col_bytes || !c->col_zero) {
    (void)hipDeviceSynchronize();
    if (c->col_buf) (void)hipFree(c->col_buf);
    c->col_buf = nullptr;
    c->col_bytes = 0;
    hipError_t e = hipMalloc(&c->col_buf, need);
    if (e != hipSuccess) return hip_fail(c, e, "column matrix hipMalloc");
    c->col_bytes = need;
    if (!c->col_zero) {  // a zero bias for the column GEMM, as long as any of its M
      const size_t zb = static_cast<size_t>(2) * 64 * 8192 * sizeof(float);
      e = hipMalloc(&c->col_zero, zb);
      if (e == hipSuccess) e = hipMemset(c->col_zero, 0, zb);
      if (e != hipSuccess) return hip_fail(c, e, "column matrix bias");
    }
  }
  ConvDev G = L;
  G.taps = 1;
  G.M = G.cout = mcol;
  G.ups = 1;
  G.crop = 0;
  G.bias = c->col_zero;
  ConvIO gio{};
  gio.x = io.x;
  gio.T_in = io.T_in;
  gio.rate_in = io.rate_in;
  gio.h_out = c->col_buf;
  voc_status st = run_conv(c, G, gio, rows, row_len, VOC_K_CONVT, s);
  if (st) return st;
  Col2imArgs a{};
  a.col = c->col_buf;
  a.T_col = io.T_in + c->mg;
  a.Cout = L.cout;
  a.s = L.ups;
  a.crop = L.crop;
  a.bias = L.bias;
  a.h_out = io.h_out;
  a.s_out = io.s_out;
  a.s_alpha = io.snake_next ? io.snake_next->alpha : nullptr;
  a.s_invden = io.snake_next ? io.snake_next->invden : nullptr;
  a.T_out = io.T_in * L.ups + c->mg;
  a.row_len = row_len;
  a.rate_in = io.rate_in;
  a.rows = rows;
  a.op = c->op;
  const double el = static_cast<double>(rows) * io.T_in * L.ups * L.cout;
  const double hs = hsz(c);  // the column matrix and h use the residual element type
  const double bytes = el * (2.0 * hs + (io.h_out ? hs : 0.0) + (io.s_out ? op_size(c->op) : 0.0));
  return launch(c, s, VOC_K_COL2IM, 0.0, bytes, "col2im launch", [&] { return launch_col2im(a, s); });
}

voc_status run_import(voc_ctx* c, const float* x, int64_t T_src, int C, const RowInfo& rows,
                      int nrows, int T, void* s_out, const SnakeDev* sn, float* h_out,
                      hipStream_t s, const SnakeDev* h_sn = nullptr) {
  ImportArgs a{};
  a.x = x;
  a.T_src = T_src;
  a.C = C;
  a.rows = rows;
  a.nrows = nrows;
  a.T = T + c->mg;
  a.T_write = T;
  a.op = c->op;
  a.s_out = s_out;
  a.s_alpha = sn ? sn->alpha : nullptr;
  a.s_invden = sn ? sn->invden : nullptr;
  a.h_out = h_out;
  a.h_scale = h_sn ? h_sn->alpha : nullptr;
  a.h_h = h_sn ? h_sn->invden : nullptr;
  const double el = static_cast<double>(nrows) * T * C;
  const double bytes = el * 4 + (s_out ? el * op_size(c->op) : 0) + (h_out ? el * hsz(c) : 0);
  return launch(c, s, VOC_K_IMPORT, 0.0, bytes, "import launch", [&] { return launch_import(a, s); });
}

// With `snake`, h is the fp16 residual stream and the head applies that
// Snake_out while loading (bf16 decoders); without, h holds Snake_out(h) in
// fp32.
voc_status run_head(voc_ctx* c, const float* h, int T, const RowInfo& rows, int nrows, int rate,
                    float* pcm, int64_t ch_stride, hipStream_t s, const SnakeDev* snake = nullptr) {
  HeadArgs a{};
  a.s_scale = snake ? snake->alpha : nullptr;
  a.s_h = snake ? snake->invden : nullptr;
  const voc_config& g = c->cfg;
  a.h = h;
  a.C = g.width[g.n_blocks];
  a.T = T + c->mg;
  a.rows = rows;
  a.nrows = nrows;
  a.rate = rate;
  a.pad = c->cfg.causal ? 6 : 3;
  a.lb = c->st_active ? a.pad : 0;
  a.nout = g.out_channels;
  a.ch_stride = ch_stride;
  a.w = c->W.head_w;
  a.bias[0] = c->W.head_bias[0];
  a.bias[1] = c->W.head_bias[1];
  a.pcm = pcm;
  a.no_tanh = c->head_no_tanh ? 1 : 0;
  // The kernel reads and writes only the kept samples of each row (their
  // count is in the row metadata last uploaded for these rows).
  double frames = static_cast<double>(nrows) * T;
  const std::vector<int>& mi = c->meta_int;
  if (mi.size() == static_cast<size_t>(5 * nrows)) {
    frames = 0.0;
    for (int r = 0; r < nrows; ++r) frames += mi[4 * nrows + r] - mi[3 * nrows + r];
  }
  const double flops = 2.0 * frames * a.C * 7 * a.nout;
  const double bytes = frames * a.C * (snake ? hsz(c) : 4) + frames * 4 * a.nout;
  return launch(c, s, VOC_K_HEAD, flops, bytes, "head launch", [&] { return launch_head(a, s); });
}

// A Snake as a launch of its own: x (fp32 residual-stream layout, C
// channels, T frames per row at `rate` frames per latent frame) into out
// (operand layout of out_op).  Alias-free configurations run the alias-free
// Snake (algorithmic work per element: two upsampled samples of six taps,
// two Snakes, one twelve-tap output, 48 flops counting an FMA as two); the
// split ablation runs the plain elementwise Snake.  Bytes: the fp32 read
// and the operand write.
voc_status run_af(voc_ctx* c, const SnakeDev& sn, const float* x, int C, int T, int rate, int rows,
                  const int* row_len, void* out, int out_op, hipStream_t s) {
  AfArgs a{};
  a.x = x;
  a.out = out;
  a.out_op = out_op;
  a.C = C;
  a.T = T + c->mg;
  a.row_len = row_len;
  a.rate = rate;
  a.scale = sn.alpha;
  a.hh = sn.invden;
  std::memcpy(a.fe, c->af_fe, sizeof(a.fe));
  std::memcpy(a.fo, c->af_fo, sizeof(a.fo));
  std::memcpy(a.fd, c->af_fd, sizeof(a.fd));
  a.rows = rows;
  a.h16 = c->op == OP_BF16 ? 1 : 0;
  const double el = static_cast<double>(rows) * T * C;
  const double hs = hsz(c);
  const double ob = op_size(out_op);  // OP_F32: fp32 (the head's input, or fp32 operands)
  if (!c->cfg.af_snake)
    return launch(c, s, VOC_K_SNAKE, 0.0, el * (hs + ob), "Snake launch",
                  [&] { return launch_snake(a, s); });
  return launch(c, s, VOC_K_AF_SNAKE, 48.0 * el, el * (hs + ob), "alias-free Snake launch",
                [&] { return launch_af_snake(a, s); });
}

// One residual unit: fused into one kernel when an instance exists for its
// width, else conv1 (epilogue: bias + Snake2 -> ubuf) and conv2 (epilogue:
// bias + residual + next Snake).  s_in holds Snake1(h) in the operand dtype,
// except when h_alt is given: then the fused kernel computes Snake1 from h
// itself (s_in unused) and writes the updated h to h_alt.
// When `next` is given, the next layer's Snake operand is written to
// *s_next: s_spare for the fused kernel (its tiles read neighbouring frames
// of s_in while others write, so it must not write in place), s_in for the
// two-kernel path (conv1 has finished reading s_in before conv2 runs).
voc_status run_res_unit(voc_ctx* c, const UnitDev& u, const void* s_in, void* s_spare, void* ubuf,
                        float* h, float* h_alt, const SnakeDev* next, void** s_next, int T, int rate,
                        int rows, const int* row_len, hipStream_t s, const SnakeDev* h_snake = nullptr,
                        bool keep_h = true) {
  const int C = u.c1.cout;
  // The large-frame tile where it still gives two workgroups per CU.
  const int bn_big = c->no_fuse ? 0 : res_unit_tile(c->op, C, true, c->terms);
  const bool big = bn_big > 0 && static_cast<int64_t>((T + bn_big - 1) / bn_big) * rows >= 2 * 256;
  const int bn = c->no_fuse ? 0 : (big ? bn_big : res_unit_tile(c->op, C, false, c->terms));
  if (s_next) *s_next = nullptr;
  if (h_alt && bn <= 0) return fail(c, VOC_DEVICE_ERROR, "no fused residual unit for this width");
  if (bn > 0) {
    void* s_out = next ? s_spare : nullptr;
    if (s_next) *s_next = s_out;
    ResUnitArgs a{};
    a.x = h_alt ? nullptr : s_in;
    a.x_from_h = h_alt ? 1 : 0;
    a.a1_scale = u.a1.alpha;
    a.a1_h = u.a1.invden;
    a.h_in = h;
    a.T = T + c->mg;
    a.C = C;
    a.row_len = row_len;
    a.rate = rate;
    a.dil = u.c1.dil;
    a.pad = (u.c1.causal ? 6 : 3) * u.c1.dil;
    a.lb = c->st_active ? a.pad : 0;
    a.w1 = u.c1.w;
    a.b1 = u.c1.bias;
    a.a2_scale = u.a2.alpha;
    a.a2_h = u.a2.invden;
    a.w2 = u.c2.w;
    a.b2 = u.c2.bias;
    a.h = h_alt ? h_alt : h;
    a.terms = c->terms;
    a.store_h = keep_h ? 1 : 0;
    a.s_out = s_out;
    a.s_scale = next ? next->alpha : nullptr;
    a.s_h = next ? next->invden : nullptr;
    a.hs_scale = h_snake ? h_snake->alpha : nullptr;
    a.hs_h = h_snake ? h_snake->invden : nullptr;
    a.n_tiles = (T + bn - 1) / bn;
    a.rows = rows;
    const double el = static_cast<double>(rows) * T * C;
    const double es = op_size(c->op) * c->terms;  // operand bytes per element
    const double flops = 2.0 * el * C * 8;
    // Reads: the operand (or h itself) and h; writes: h if kept, the next operand.
    const double hs = hsz(c);
    // (With two-term operands the operand tensors and the packed weights are twice as large.)
    const double bytes = el * ((h_alt ? hs : es + hs) + (keep_h ? hs : 0) + (s_out ? es : 0)) + 8.0 * C * C * es;
    const int op = c->op;
    return launch(c, s, VOC_K_RES_FUSED, flops, bytes, "residual unit launch",
                  [&] { return launch_res_unit(op, a, big, s); });
  }
  void* s_out = next ? const_cast<void*>(s_in) : nullptr;
  if (s_next) *s_next = s_out;
  ConvIO io{};
  io.x = s_in;
  io.T_in = T;
  io.rate_in = rate;
  io.s_out = ubuf;
  io.snake_next = &u.a2;
  voc_status st = run_conv(c, u.c1, io, rows, row_len, VOC_K_RES_K7, s);
  if (st) return st;
  io = ConvIO{};
  io.x = ubuf;
  io.T_in = T;
  io.rate_in = rate;
  io.h_out = keep_h ? h : nullptr;
  io.res = h;
  io.snake_next = next;
  io.s_out = s_out;
  io.h_snake = h_snake;
  return run_conv(c, u.c2, io, rows, row_len, VOC_K_RES_K1, s);
}

// One residual unit with alias-free Snakes (four launches; the Snakes read
// neighbouring frames, so neither fits a GEMM epilogue or the fused unit):
//   AF1(h) -> s_buf;  conv1 -> h2 (fp32);  AF2(h2) -> u_buf;  h += conv2(u_buf).
voc_status run_res_unit_af(voc_ctx* c, const UnitDev& u, float* h, float* h2, void* s_buf, void* u_buf,
                           int T, int rate, int rows, const int* row_len, hipStream_t s) {
  const int C = u.c1.cout;
  voc_status st = run_af(c, u.a1, h, C, T, rate, rows, row_len, s_buf, c->op, s);
  if (st) return st;
  ConvIO io{};
  io.x = s_buf;
  io.T_in = T;
  io.rate_in = rate;
  io.h_out = h2;
  st = run_conv(c, u.c1, io, rows, row_len, VOC_K_RES_K7, s);
  if (st) return st;
  st = run_af(c, u.a2, h2, C, T, rate, rows, row_len, u_buf, c->op, s);
  if (st) return st;
  io = ConvIO{};
  io.x = u_buf;
  io.T_in = T;
  io.rate_in = rate;
  io.h_out = h;
  io.res = h;
  return run_conv(c, u.c2, io, rows, row_len, VOC_K_RES_K1, s);
}

const SnakeDev* next_snake(const Weights& W, int b, int r, int nb, int nr) {
  if (r + 1 < nr) return &W.blocks[b].units[r + 1].a1;
  if (b + 1 < nb) return &W.blocks[b + 1].act;
  return nullptr;
}

// The whole decoder over `rows` rows of T latent frames (already imported
// into xlat).  *h_last receives the buffer holding the last residual stream
// (B.h or B.h2).
voc_status run_stack(voc_ctx* c, const Bufs& B, int rows, int T, hipStream_t s, float** h_last) {
  const voc_config& g = c->cfg;
  const Weights& W = c->W;
  const int nb = g.n_blocks, nr = g.n_res;
  int cur = 0;
  // Stream chunks: before each layer with context, its input's margin gets
  // the context carried from the previous chunk and the new context is saved
  // (layer index li in the order of voc_ctx::st_layers).
  int li = 0;
  auto xchg = [&](const void* buf, int64_t frames) -> voc_status {
    if (!c->st_active) return VOC_OK;
    const voc_ctx::LayerState& L = c->st_layers[li++];
    LayerStateArgs a{};
    a.buf = static_cast<unsigned char*>(const_cast<void*>(buf));
    a.plane_bytes = (c->mg + frames) * L.row_bytes;
    a.planes = static_cast<int64_t>(rows) * L.planes_per_row;
    a.ctx = L.ctx;
    a.Tr = static_cast<int>(frames);
    a.row_bytes = L.row_bytes;
    a.old_state = static_cast<const unsigned char*>(c->st_mem) + L.off[c->st_par];
    a.new_state = static_cast<unsigned char*>(c->st_mem) + L.off[c->st_par ^ 1];
    const double bytes = 3.0 * a.planes * a.ctx * L.row_bytes;
    return launch(c, s, VOC_K_IMPORT, 0.0, bytes, "stream state launch",
                  [&] { return launch_layer_state(a, s); });
  };
  ConvIO io{};
  const void* x_in = B.xlat;
  if (W.in_proj.cout > 0) {  // dec_in_proj: operand for conv_in, no activation between
    io.x = B.xlat;
    io.T_in = T;
    io.rate_in = 1;
    io.s_out = B.u;
    voc_status st = run_conv(c, W.in_proj, io, rows, B.rows.len, VOC_K_IN_PROJ, s);
    if (st) return st;
    x_in = B.u;
  }
  io = ConvIO{};
  io.x = x_in;
  io.T_in = T;
  io.rate_in = 1;
  io.h_out = B.h;
  io.s_out = B.s[cur];
  io.snake_next = &W.blocks[0].act;
  voc_status st = xchg(x_in, T);
  if (st) return st;
  st = run_conv(c, W.conv_in, io, rows, B.rows.len, VOC_K_CONV_IN, s);
  if (st) return st;
  int t = T, rate = 1;
  float* hc = B.h;   // current residual stream
  float* ho = B.h2;  // the other buffer (units with the operand from h)
  for (int b = 0; b < nb; ++b) {
    const BlockDev& blk = W.blocks[b];
    const bool xh = unit_xh(c, g.width[b + 1]);
    io = ConvIO{};
    io.x = B.s[cur];
    io.T_in = t;
    io.rate_in = rate;
    io.h_out = hc;
    if (!xh) {  // else the first unit computes its Snake operand from h
      io.s_out = B.s[cur ^ 1];
      io.snake_next = &blk.units[0].a1;
    }
    st = xchg(B.s[cur], t);
    if (st) return st;
    st = run_convt(c, blk.ct, io, rows, B.rows.len, s);
    if (st) return st;
    if (!xh) cur ^= 1;
    t *= g.stride[b];
    rate *= g.stride[b];
    for (int r = 0; r < nr; ++r) {
      void* s_next = nullptr;
      // The last unit stores the head's Snake of h: nothing else reads h.
      const SnakeDev* hs = (b == nb - 1 && r == nr - 1 && !head_snake_at_load(c)) ? &W.head_act : nullptr;
      // The last unit of any other block feeds the next block only through
      // its Snake operand; its h is never read again.
      const bool keep_h = !(r == nr - 1 && b < nb - 1);
      // Within a block of such units only the last one writes an operand
      // tensor (the next block's ConvTranspose1d input).
      const SnakeDev* next = (xh && r + 1 < nr) ? nullptr : next_snake(W, b, r, nb, nr);
      st = xchg(xh ? static_cast<const void*>(hc) : B.s[cur], t);  // conv1's input
      if (st) return st;
      st = run_res_unit(c, blk.units[r], xh ? nullptr : B.s[cur], B.s[cur ^ 1], B.u, hc,
                        xh ? ho : nullptr, next, &s_next, t, rate, rows, B.rows.len, s, hs, keep_h);
      if (st) return st;
      if (s_next == B.s[cur ^ 1]) cur ^= 1;
      if (xh && keep_h) std::swap(hc, ho);
    }
  }
  *h_last = hc;
  return xchg(hc, t);  // the head's input
}

// The alias-free decoder (TensorSharp minimax-h3 page, audio VAE): producers
// write the residual stream h only, and every Snake is an alias-free Snake
// launch that writes the next GEMM's operand.  The head's input, AF(h), goes
// to h2 in fp32; *h_last receives h2.  The split ablation runs the same
// sequence with plain Snake launches (the standalone Snake stage).
voc_status run_stack_af(voc_ctx* c, const Bufs& B, int rows, int T, hipStream_t s, float** h_last) {
  const voc_config& g = c->cfg;
  const Weights& W = c->W;
  ConvIO io{};
  const void* x_in = B.xlat;
  voc_status st;
  if (W.in_proj.cout > 0) {
    io.x = B.xlat;
    io.T_in = T;
    io.rate_in = 1;
    io.s_out = B.u;
    st = run_conv(c, W.in_proj, io, rows, B.rows.len, VOC_K_IN_PROJ, s);
    if (st) return st;
    x_in = B.u;
  }
  io = ConvIO{};
  io.x = x_in;
  io.T_in = T;
  io.rate_in = 1;
  io.h_out = B.h;
  st = run_conv(c, W.conv_in, io, rows, B.rows.len, VOC_K_CONV_IN, s);
  if (st) return st;
  int t = T, rate = 1;
  for (int b = 0; b < g.n_blocks; ++b) {
    const BlockDev& blk = W.blocks[b];
    st = run_af(c, blk.act, B.h, g.width[b], t, rate, rows, B.rows.len, B.s[0], c->op, s);
    if (st) return st;
    io = ConvIO{};
    io.x = B.s[0];
    io.T_in = t;
    io.rate_in = rate;
    io.h_out = B.h;  // the Snake above has consumed h
    st = run_convt(c, blk.ct, io, rows, B.rows.len, s);
    if (st) return st;
    t *= g.stride[b];
    rate *= g.stride[b];
    for (int r = 0; r < g.n_res; ++r) {
      st = run_res_unit_af(c, blk.units[r], B.h, B.h2, B.s[0], B.u, t, rate, rows, B.rows.len, s);
      if (st) return st;
    }
  }
  st = run_af(c, W.head_act, B.h, g.width[g.n_blocks], t, rate, rows, B.rows.len, B.h2, OP_F32, s);
  if (st) return st;
  *h_last = B.h2;
  return VOC_OK;
}

void free_weights(Weights& W) {
  for (void* p : W.allocs) (void)hipFree(p);
  W = Weights{};
}

}  // namespace

// =================================================================== ABI


VOC_API voc_status vocoder_create(const voc_config* cfg, int hip_device, voc_ctx** out) {
  if (!out) return fail(nullptr, VOC_INVALID_PARAMS, "out is NULL");
  *out = nullptr;
  std::string why;
  if (validate(cfg, &why) != VOC_OK) return fail(nullptr, VOC_INVALID_PARAMS, why);
  int ndev = 0;
  hipError_t e = hipGetDeviceCount(&ndev);
  if (e != hipSuccess || ndev <= 0) return fail(nullptr, VOC_DEVICE_ERROR, "no HIP device");
  if (hip_device < 0 || hip_device >= ndev) return fail(nullptr, VOC_INVALID_PARAMS, "bad device index");
  e = hipSetDevice(hip_device);
  if (e != hipSuccess) return fail(nullptr, VOC_DEVICE_ERROR, "hipSetDevice failed");
  // This device's copy of the no-allocation scratch array: its address is
  // taken once per device, with the device current, and kept.
  void* scratch_ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (hip_device < kMaxDevices && !g_scratch_ptr[hip_device]) {
      e = hipGetSymbolAddress(&g_scratch_ptr[hip_device], HIP_SYMBOL(scratch));
      if (e != hipSuccess) {
        g_scratch_ptr[hip_device] = nullptr;
        return fail(nullptr, VOC_DEVICE_ERROR,
                    std::string("hipGetSymbolAddress of the scratch array: ") + hipGetErrorString(e));
      }
    }
    if (hip_device < kMaxDevices) scratch_ptr = g_scratch_ptr[hip_device];
  }
  voc_ctx* c = new (std::nothrow) voc_ctx();
  if (!c) return fail(nullptr, VOC_OOM, "host allocation failed");
  c->scratch = scratch_ptr;
  c->cfg = *cfg;
  c->device = hip_device;
  c->op = cfg->dtype == VOC_F32 ? OP_F32 : OP_BF16;
  c->hop = total_stride(*cfg);
  compute_halos(*cfg, &c->halo_l, &c->halo_r);
  if (cfg->af_snake) design_af_filter(c->af_fe, c->af_fo, c->af_fd);
  if (const char* cap = std::getenv("VOC_MAX_WORKSPACE_BYTES")) c->ws_cap = std::strtoull(cap, nullptr, 10);
  // Ablation only: VOC_VARIANT_{CONV_IN,CONVT,RES_K7,RES_K1}=<tile family index>.
  const char* names[4] = {"VOC_VARIANT_CONV_IN", "VOC_VARIANT_CONVT", "VOC_VARIANT_RES_K7",
                          "VOC_VARIANT_RES_K1"};
  for (int k = 0; k < 4; ++k)
    if (const char* v = std::getenv(names[k])) c->force_variant[k] = std::atoi(v);
  if (const char* v = std::getenv("VOC_NO_FUSED_RES")) c->no_fuse = std::atoi(v) != 0;
  // Test switch: VOC_MAX_ROW_FRAMES lowers the row-frame limit, so that the
  // automatic time tiling of long rows can be exercised at small sizes.
  if (const char* v = std::getenv("VOC_MAX_ROW_FRAMES")) c->frames_cap = std::atoll(v);
  if (const char* v = std::getenv("VOC_CONV_M_FAST")) c->m_order = std::atoi(v) != 0;
  // Ablation only: 0 makes every fused unit read an operand tensor written by its producer.
  if (const char* v = std::getenv("VOC_RU_OPERAND_FROM_H")) c->ru_xh = std::atoi(v) != 0;
  // Ablation only: 1 runs every Snake of a plain decode as a launch of its own
  // (producers write h only), to measure the standalone Snake stage.
  if (const char* v = std::getenv("VOC_SPLIT_SNAKE")) c->split_snake = std::atoi(v) != 0 && !cfg->causal;
  // Ablation only: 1 runs every ConvTranspose1d as a GEMM into a column
  // matrix followed by a col2im overlap-add (the pages' lowering).
  if (const char* v = std::getenv("VOC_CONVT_COL2IM")) c->col2im = std::atoi(v) != 0 && !cfg->causal;
  // Ablation only: 1 makes vocoder_decode's head store the pre-tanh sums and
  // applies tanh in a pass of its own over the pcm (untiled decodes without a
  // cancel hook; otherwise the head applies it as usual).
  if (const char* v = std::getenv("VOC_SPLIT_TANH")) c->split_tanh = std::atoi(v) != 0;
  // Two-term operands: every kernel that writes a matrix-core operand in a
  // decode writes both terms; the standalone Snake and col2im ablations
  // write one and are off for such a decoder.
  c->terms = cfg->operand_terms == 2 ? 2 : 1;
  if (c->terms == 2) c->split_snake = c->col2im = false;
  *out = c;
  return VOC_OK;
}

VOC_API voc_status vocoder_load_weights(voc_ctx* c, const voc_tensor* t, int n) {
  if (!c) return VOC_INVALID_PARAMS;
  if (!t || n <= 0) return fail(c, VOC_INVALID_PARAMS, "no tensors");
  const voc_config& g = c->cfg;
  auto exp = expected_tensors(g);
  std::map<std::string, const voc_tensor*> got;
  for (int i = 0; i < n; ++i) {
    if (!t[i].name || !t[i].data) return fail(c, VOC_INVALID_PARAMS, "tensor with NULL name or data");
    if (t[i].ndim < 0 || t[i].ndim > 4) return fail(c, VOC_BAD_WEIGHTS, std::string("bad ndim: ") + t[i].name);
    auto it = exp.find(t[i].name);
    if (it == exp.end()) return fail(c, VOC_BAD_WEIGHTS, std::string("unknown tensor: ") + t[i].name);
    if (got.count(t[i].name)) return fail(c, VOC_BAD_WEIGHTS, std::string("duplicate tensor: ") + t[i].name);
    if (squeeze(t[i].shape, t[i].ndim) != it->second.shape)
      return fail(c, VOC_BAD_WEIGHTS, std::string("shape mismatch: ") + t[i].name);
    got[t[i].name] = &t[i];
  }
  for (auto& kv : exp)
    if (!got.count(kv.first)) return fail(c, VOC_BAD_WEIGHTS, "missing tensor: " + kv.first);
  // Small tensors are checked on the host; weight_v through its norm.
  for (auto& kv : got) {
    const std::string& nm = kv.first;
    if (nm.size() > 9 && nm.compare(nm.size() - 9, 9, ".weight_v") == 0) continue;
    if (!all_finite(kv.second->data, numel(*kv.second)))
      return fail(c, VOC_BAD_WEIGHTS, "non-finite value in " + nm);
  }

  Weights W;
  std::vector<void*> staging;  // v, g and norm buffers, freed after the fold
  const int op = c->op;
  std::vector<double*> norm_bufs;
  std::vector<std::pair<std::string, int64_t>> norm_names;
  auto dalloc = [&](size_t bytes, void** p) -> voc_status {
    hipError_t e = hipMalloc(p, bytes);
    if (e != hipSuccess) {
      *p = nullptr;
      return hip_fail(c, e, "weight hipMalloc");
    }
    W.allocs.push_back(*p);
    return VOC_OK;
  };
  auto upload = [&](const float* h, size_t count, float** d, bool stage = false) -> voc_status {
    voc_status st = dalloc(count * 4, reinterpret_cast<void**>(d));
    if (st) return st;
    if (stage) {
      W.allocs.pop_back();
      staging.push_back(*d);
    }
    hipError_t e = hipMemcpy(*d, h, count * 4, hipMemcpyHostToDevice);
    return e == hipSuccess ? VOC_OK : hip_fail(c, e, "weight upload");
  };
  // Snake parameters as the kernels use them: scale = alpha / pi and
  // h = 1 / (2 (den + 1e-9)), den = alpha (Snake) or beta (SnakeBeta).
  auto snake = [&](const std::string& p, int ch, SnakeDev* sd) -> voc_status {
    const float* a = got[p + ".alpha"]->data;
    const float* b = g.act == VOC_SNAKE_BETA ? got[p + ".beta"]->data : nullptr;
    std::vector<float> sc(ch), hh(ch);
    for (int i = 0; i < ch; ++i) {
      double av = a[i], dv = b ? b[i] : a[i];
      if (g.snake_log_params) av = std::exp(av), dv = std::exp(dv);
      sc[i] = static_cast<float>(av / M_PI);
      hh[i] = static_cast<float>(0.5 / (dv + 1e-9));
      if (!std::isfinite(sc[i]) || !std::isfinite(hh[i]))
        return fail(c, VOC_BAD_WEIGHTS, "Snake parameter gives a non-finite value in " + p);
    }
    voc_status st = upload(sc.data(), ch, &sd->alpha);
    if (st) return st;
    return upload(hh.data(), ch, &sd->invden);
  };
  // Fold one conv: v is uploaded to a staging buffer, folded into the packed layout.
  // plain: the tensor is p.weight, used as stored (no weight norm).
  // cin_alloc > cin: packed with cin_alloc input channels, the extra ones zero.
  // copies = 2: the packed tensor is stored twice in a row (two-term operands:
  // the low-term input channels meet the same weights).
  auto fold = [&](const std::string& p, int kind, int cin, int cout, int k, int stride,
                  void** out_w, float** out_bias, bool plain = false, int cin_alloc = 0,
                  int copies = 1) -> voc_status {
    const voc_tensor* tv = got[plain ? p + ".weight" : p + ".weight_v"];
    const int64_t cnt = numel(*tv);
    const int64_t d0 = kind == PACK_CONVT ? cin : cout;
    float *dv = nullptr, *dg = nullptr;
    voc_status st = upload(tv->data, cnt, &dv, true);
    if (st) return st;
    if (!plain) {
      st = upload(got[p + ".weight_g"]->data, d0, &dg, true);
      if (st) return st;
    }
    double* dn = nullptr;
    st = dalloc(d0 * sizeof(double), reinterpret_cast<void**>(&dn));
    if (st) return st;
    W.allocs.pop_back();
    staging.push_back(dn);
    const size_t es = kind == PACK_HEAD ? 4 : op_size(op);
    size_t out_elems = static_cast<size_t>(cnt);
    if (kind == PACK_DOWN) out_elems = static_cast<size_t>(cout) * cin * 2 * stride;  // 2 taps x s phases
    if (cin_alloc > cin) out_elems = static_cast<size_t>(cout) * k * cin_alloc;
    st = dalloc(out_elems * es * copies, out_w);
    if (st) return st;
    if (out_elems != static_cast<size_t>(cnt)) {  // entries no weight maps to stay zero
      hipError_t e = hipMemset(*out_w, 0, out_elems * es);
      if (e != hipSuccess) return hip_fail(c, e, "weight clear");
    }
    FoldArgs fa{};
    fa.v = dv;
    fa.g = dg;
    fa.d0 = d0;
    fa.rest = cnt / d0;
    fa.kind = kind;
    fa.op = kind == PACK_HEAD ? OP_F32 : op;
    fa.round_bf16 = kind == PACK_HEAD && op == OP_BF16;
    fa.cin = cin;
    fa.cout = cout;
    fa.k = k;
    fa.stride = stride;
    fa.out = *out_w;
    fa.norms = dn;
    hipError_t e = launch_fold(fa, nullptr);
    if (e != hipSuccess) return hip_fail(c, e, "fold launch");
    for (int k2 = 1; k2 < copies; ++k2) {
      e = hipMemcpy(static_cast<char*>(*out_w) + k2 * out_elems * es, *out_w, out_elems * es,
                    hipMemcpyDeviceToDevice);
      if (e != hipSuccess) return hip_fail(c, e, "weight copy");
    }
    if (!plain) {  // ||v|| must be positive and finite
      norm_bufs.push_back(dn);
      norm_names.push_back({p, d0});
    }
    if (out_bias) return upload(got[p + ".bias"]->data, cout, out_bias);
    return VOC_OK;
  };

  auto build = [&]() -> voc_status {
    voc_status st;
    if (g.in_proj > 0) {
      ConvDev& ip = W.in_proj;
      ip.cin = g.latent_channels;
      ip.cout = ip.M = g.in_proj;
      ip.taps = 1;
      st = fold("dec_in_proj", PACK_CONV, ip.cin, ip.cout, 1, 1, &ip.w, &ip.bias, true);
      if (st) return st;
    }
    ConvDev& ci = W.conv_in;
    ci.cin = g.in_proj > 0 ? g.in_proj : g.latent_channels;
    ci.cout = ci.M = g.width[0];
    ci.taps = 7;
    ci.causal = g.causal;
    st = fold("conv_in", PACK_CONV, ci.cin, ci.cout, 7, 1, &ci.w, &ci.bias);
    if (st) return st;
    W.blocks.resize(g.n_blocks);
    for (int b = 0; b < g.n_blocks; ++b) {
      const std::string p = "blocks." + std::to_string(b);
      BlockDev& blk = W.blocks[b];
      const int cin = g.width[b], cout = g.width[b + 1], s = g.stride[b];
      st = snake(p + ".snake1", cin, &blk.act);
      if (st) return st;
      blk.ct.cin = cin;
      blk.ct.cout = cout;
      blk.ct.taps = 2;
      blk.ct.ups = s;
      blk.ct.crop = g.causal ? 0 : (s + 1) / 2;  // causal: keep full[0, T*s)
      blk.ct.M = s * cout;
      blk.ct.terms = c->terms;
      st = fold(p + ".conv_t1", PACK_CONVT, cin, cout, 2 * s, s, &blk.ct.w, &blk.ct.bias, false, 0, c->terms);
      if (st) return st;
      blk.units.resize(g.n_res);
      for (int r = 0; r < g.n_res; ++r) {
        const std::string q = p + ".res_units." + std::to_string(r);
        UnitDev& u = blk.units[r];
        st = snake(q + ".snake1", cout, &u.a1);
        if (st) return st;
        st = snake(q + ".snake2", cout, &u.a2);
        if (st) return st;
        u.c1.cin = u.c1.cout = u.c1.M = cout;
        u.c1.taps = 7;
        u.c1.dil = g.dilation[r];
        u.c1.causal = g.causal;
        u.c1.terms = u.c2.terms = c->terms;
        st = fold(q + ".conv1", PACK_CONV, cout, cout, 7, 1, &u.c1.w, &u.c1.bias, false, 0, c->terms);
        if (st) return st;
        u.c2.cin = u.c2.cout = u.c2.M = cout;
        u.c2.taps = 1;
        st = fold(q + ".conv2", PACK_CONV, cout, cout, 1, 1, &u.c2.w, &u.c2.bias, false, 0, c->terms);
        if (st) return st;
      }
    }
    st = snake("snake_out", g.width[g.n_blocks], &W.head_act);
    if (st) return st;
    void* hw = nullptr;
    st = fold("conv_out", PACK_HEAD, g.width[g.n_blocks], g.out_channels, 7, 1, &hw, nullptr);
    if (st) return st;
    W.head_w = static_cast<float*>(hw);
    for (int o = 0; o < g.out_channels; ++o) W.head_bias[o] = got["conv_out.bias"]->data[o];
    if (g.enc_width[0] > 0) {
      const int* E = g.enc_width;
      const int CHn = op_chunk(op);
      EncoderDev& en = W.enc;
      en.conv_in.cin = CHn;  // one real channel in a zero-padded chunk
      en.conv_in.cout = en.conv_in.M = E[0];
      en.conv_in.taps = 7;
      st = fold("encoder.conv_in", PACK_CONV, 1, E[0], 7, 1, &en.conv_in.w, &en.conv_in.bias, false, CHn);
      if (st) return st;
      en.blocks.resize(g.n_blocks);
      for (int b = 0; b < g.n_blocks; ++b) {
        const std::string q = "encoder.blocks." + std::to_string(b);
        EncBlockDev& eb = en.blocks[b];
        eb.units.resize(g.n_res);
        for (int r = 0; r < g.n_res; ++r) {
          const std::string u = q + ".res_units." + std::to_string(r);
          UnitDev& ud = eb.units[r];
          st = snake(u + ".snake1", E[b], &ud.a1);
          if (!st) st = snake(u + ".snake2", E[b], &ud.a2);
          if (st) return st;
          ud.c1.cin = ud.c1.cout = ud.c1.M = E[b];
          ud.c1.taps = 7;
          ud.c1.dil = g.dilation[r];
          st = fold(u + ".conv1", PACK_CONV, E[b], E[b], 7, 1, &ud.c1.w, &ud.c1.bias);
          if (st) return st;
          ud.c2.cin = ud.c2.cout = ud.c2.M = E[b];
          ud.c2.taps = 1;
          st = fold(u + ".conv2", PACK_CONV, E[b], E[b], 1, 1, &ud.c2.w, &ud.c2.bias);
          if (st) return st;
        }
        st = snake(q + ".snake", E[b], &eb.act);
        if (st) return st;
        const int sb = g.stride[g.n_blocks - 1 - b];
        eb.down.cin = E[b];
        eb.down.cout = eb.down.M = E[b + 1];
        eb.down.taps = 2;
        eb.down.down = sb;
        st = fold(q + ".down", PACK_DOWN, E[b], E[b + 1], 2 * sb, sb, &eb.down.w, &eb.down.bias);
        if (st) return st;
      }
      const int En = E[g.n_blocks];
      st = snake("encoder.snake_out", En, &en.out_act);
      if (st) return st;
      en.conv_out.cin = en.conv_out.cout = en.conv_out.M = En;
      en.conv_out.taps = 3;
      st = fold("encoder.conv_out", PACK_CONV, En, En, 3, 1, &en.conv_out.w, &en.conv_out.bias);
      if (st) return st;
      en.proj.cin = En;
      en.proj.cout = en.proj.M = g.latent_channels;
      en.proj.taps = 1;
      st = fold("encoder.proj", PACK_CONV, En, g.latent_channels, 1, 1, &en.proj.w, &en.proj.bias);
      if (st) return st;
    }
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(c, e, "fold");
    for (size_t i = 0; i < norm_bufs.size(); ++i) {
      std::vector<double> nv(norm_names[i].second);
      e = hipMemcpy(nv.data(), norm_bufs[i], nv.size() * sizeof(double), hipMemcpyDeviceToHost);
      if (e != hipSuccess) return hip_fail(c, e, "norm readback");
      for (double x : nv)
        if (!(x > 0.0) || !std::isfinite(x))
          return fail(c, VOC_BAD_WEIGHTS, "zero or non-finite ||v|| in " + norm_names[i].first);
    }
    return VOC_OK;
  };
  voc_status st = build();
  (void)hipDeviceSynchronize();
  for (void* q : staging) (void)hipFree(q);
  if (st != VOC_OK) {
    free_weights(W);
    return st;
  }
  free_weights(c->W);
  c->W = W;
  c->loaded = true;
  c->err.clear();
  return VOC_OK;
}

VOC_API int64_t vocoder_output_length(const voc_ctx* c, int64_t T) {
  if (!c || T < 0) return -1;
  return T * c->hop;
}

namespace {
// The cancel hook's answer (false without a hook).
bool cancel_requested(voc_ctx* c) { return c->cancel_fn && c->cancel_fn(c->cancel_user) != 0; }

voc_status cancelled(voc_ctx* c) { return fail(c, VOC_CANCELLED, "cancelled by the cancel hook"); }

// One batched decode of `rows` rows read from latent [*, C, T_src] through
// the row metadata (dst, ints = len | src_b | start | keep_lo | keep_hi),
// which is uploaded unless `key` matches what the workspace already holds.
// Output channel o of row r starts at pcm[dst[r] + o * ch_stride].
voc_status decode_batch(voc_ctx* c, const float* latent, int64_t T_src, int64_t rows, int T_alloc,
                        std::vector<int64_t>&& dst, std::vector<int>&& ints,
                        std::vector<int64_t>&& key, float* pcm, int64_t ch_stride, hipStream_t s) {
  const voc_config& g = c->cfg;
  const Plan p = make_plan(c, static_cast<int>(rows), T_alloc);
  voc_status st = ensure_ws(c, p.bytes);
  if (st) return st;
  if (c->ws_override || c->rows_key != key) {
    // The scratch is shared by every context on the device: its metadata
    // is uploaded by every call and never cached.
    st = upload_rows(c, p, std::move(dst), std::move(ints), s);
    if (st) return st;
    if (c->ws_override)
      c->rows_key.clear();
    else
      c->rows_key = std::move(key);
  }
  const Bufs Bf = bufs(c, p);
  st = run_import(c, latent, T_src, g.latent_channels, Bf.rows, static_cast<int>(rows), T_alloc, Bf.xlat,
                  nullptr, nullptr, s);
  if (st) return st;
  float* h_last = nullptr;
  st = g.af_snake || c->split_snake ? run_stack_af(c, Bf, static_cast<int>(rows), T_alloc, s, &h_last)
                                    : run_stack(c, Bf, static_cast<int>(rows), T_alloc, s, &h_last);
  if (st) return st;
  return run_head(c, h_last, static_cast<int>(T_alloc * c->hop), Bf.rows, static_cast<int>(rows),
                  static_cast<int>(c->hop), pcm, ch_stride, s, head_snake_at_load(c));
}

// decode_batch over the rows in groups of `group` rows (all at once when
// group >= rows).  With a cancel hook, the hook is polled before every group
// and the stream is synchronized after each, so a cancel lands between
// groups of finished rows.  Rows are independent, so grouping changes no
// output bit.
voc_status decode_rows(voc_ctx* c, const float* latent, int64_t T_src, int64_t rows, int T_alloc,
                       std::vector<int64_t>&& dst, std::vector<int>&& ints,
                       std::vector<int64_t>&& key, float* pcm, int64_t ch_stride, hipStream_t s,
                       int64_t group) {
  if (group >= rows && !c->cancel_fn)
    return decode_batch(c, latent, T_src, rows, T_alloc, std::move(dst), std::move(ints), std::move(key),
                        pcm, ch_stride, s);
  for (int64_t r0 = 0; r0 < rows; r0 += group) {
    if (cancel_requested(c)) return cancelled(c);
    const int64_t n = std::min(group, rows - r0);
    std::vector<int64_t> gd(dst.begin() + r0, dst.begin() + r0 + n);
    std::vector<int> gi(5 * n);
    for (int f = 0; f < 5; ++f)
      std::copy(ints.begin() + f * rows + r0, ints.begin() + f * rows + r0 + n, gi.begin() + f * n);
    std::vector<int64_t> gk = key;
    gk.push_back(r0);
    gk.push_back(n);
    voc_status st = decode_batch(c, latent, T_src, n, T_alloc, std::move(gd), std::move(gi), std::move(gk),
                                 pcm, ch_stride, s);
    if (st) return st;
    if (c->cancel_fn) {
      const hipError_t e = hipStreamSynchronize(s);
      if (e != hipSuccess) return hip_fail(c, e, "stream synchronize between groups");
    }
  }
  return VOC_OK;
}

}  // namespace

namespace {
// Argument checks shared by vocoder_decode and vocoder_decode_noalloc.
voc_status check_decode_args(voc_ctx* c, const float* latent, int64_t B, int64_t T, const float* pcm) {
  if (!latent || !pcm) return fail(c, VOC_INVALID_PARAMS, "NULL latent or pcm");
  if ((reinterpret_cast<uintptr_t>(latent) | reinterpret_cast<uintptr_t>(pcm)) & 15)
    return fail(c, VOC_INVALID_PARAMS, "latent and pcm must be 16-byte aligned");
  if (B <= 0 || T <= 0) return fail(c, VOC_INVALID_PARAMS, "B and T must be positive");
  if (T * c->hop > (int64_t(1) << 31) - 1) return fail(c, VOC_INVALID_PARAMS, "T*hop exceeds 2^31-1");
  if (!c->loaded) return fail(c, VOC_NOT_LOADED, "weights not loaded");
  return VOC_OK;
}

// The rows of a decode of B rows of T latent frames: whole rows (tiled ==
// false, F == T), or tiles of F latent frames with the exact halos, b-major.
// Fills the row metadata (dst, ints = len | src_b | start | keep_lo |
// keep_hi) and the frames each row allocates.
voc_status decode_row_plan(voc_ctx* c, int64_t B, int64_t T, int64_t F, bool tiled, int64_t* rows_out,
                           int* T_alloc_out, std::vector<int64_t>* dst_out, std::vector<int>* ints_out) {
  const voc_config& g = c->cfg;
  const int64_t ntile = (T + F - 1) / F;
  const int64_t rows = B * ntile;
  if (rows > 65535) return fail(c, VOC_INVALID_PARAMS, "too many rows (B * tiles > 65535)");
  const int HL = tiled ? c->halo_l : 0;
  const int HR = tiled ? c->halo_r : 0;
  std::vector<int64_t> dst(rows);
  std::vector<int> ints(5 * rows);
  for (int64_t b = 0; b < B; ++b)
    for (int64_t k = 0; k < ntile; ++k) {
      const int64_t r = b * ntile + k;
      const int64_t t0 = k * F, t1 = std::min(T, t0 + F);
      const int64_t a = std::max<int64_t>(0, t0 - HL), e = std::min(T, t1 + HR);
      ints[r] = static_cast<int>(e - a);                          // len
      ints[rows + r] = static_cast<int>(b);                       // src_b
      ints[2 * rows + r] = static_cast<int>(a);                   // start
      ints[3 * rows + r] = static_cast<int>((t0 - a) * c->hop);   // keep_lo
      ints[4 * rows + r] = static_cast<int>((t1 - a) * c->hop);   // keep_hi
      dst[r] = (b * g.out_channels * T + t0) * c->hop;
    }
  *rows_out = rows;
  *T_alloc_out = static_cast<int>(std::min<int64_t>(T, F + HL + HR));
  *dst_out = std::move(dst);
  *ints_out = std::move(ints);
  return VOC_OK;
}

// Tile frames of a decode: the configured tile_frames, else whole rows when
// the GEMMs can address them, else the largest tile whose halos still fit.
voc_status decode_tiles(voc_ctx* c, int64_t T, int64_t* F_out, bool* tiled_out) {
  const voc_config& g = c->cfg;
  const int64_t max_frames = row_frames_limit(c);
  int64_t F = g.tile_frames > 0 ? g.tile_frames : T;
  bool tiled = g.tile_frames > 0;
  if (!tiled && T > max_frames) {
    F = max_frames - c->halo_l - c->halo_r;
    tiled = true;
  }
  if (tiled && F + c->halo_l + c->halo_r > max_frames)
    return fail(c, VOC_INVALID_PARAMS, "tile_frames plus the halos exceed the frames the GEMMs can address "
                                       "(voc_config_max_frames)");
  *F_out = F;
  *tiled_out = tiled;
  return VOC_OK;
}
}  // namespace

VOC_API voc_status vocoder_decode(voc_ctx* c, const float* latent, int64_t B, int64_t T, float* pcm,
                                  void* stream) {
  if (!c) return VOC_INVALID_PARAMS;
  voc_status st = check_decode_args(c, latent, B, T, pcm);
  if (st) return st;
  // Rows: whole rows, or tiles of tile_frames latent frames with halos.
  // Untiled rows beyond what the GEMMs can address are tiled here, with
  // the largest tile whose halos still fit (the same samples, bit for bit).
  int64_t F = 0, rows = 0;
  bool tiled = false;
  st = decode_tiles(c, T, &F, &tiled);
  if (st) return st;
  int T_alloc = 0;
  std::vector<int64_t> dst;
  std::vector<int> ints;
  st = decode_row_plan(c, B, T, F, tiled, &rows, &T_alloc, &dst, &ints);
  if (st) return st;
  const int64_t group = c->cancel_fn ? c->cancel_group : rows;
  const bool split_tanh = c->split_tanh && !tiled && !c->cancel_fn;
  c->head_no_tanh = split_tanh;
  st = decode_rows(c, latent, T, rows, T_alloc, std::move(dst), std::move(ints), {0, B, T, rows}, pcm,
                   T * c->hop, static_cast<hipStream_t>(stream), group);
  c->head_no_tanh = false;
  if (st || !split_tanh) return st;
  const int64_t n = B * c->cfg.out_channels * T * c->hop;
  return launch(c, static_cast<hipStream_t>(stream), VOC_K_TANH, 0.0, 8.0 * static_cast<double>(n),
                "tanh launch", [&] { return launch_tanh(pcm, n, static_cast<hipStream_t>(stream)); });
}

VOC_API voc_status vocoder_decode_noalloc(voc_ctx* c, const float* latent, int64_t B, int64_t T, float* pcm,
                                          void* stream) {
  if (!c) return VOC_INVALID_PARAMS;
  voc_status st = check_decode_args(c, latent, B, T, pcm);
  if (st) return st;
  if (!c->scratch) return fail(c, VOC_DEVICE_ERROR, "no scratch array on this device");
  int64_t F = 0;
  bool tiled = false;
  st = decode_tiles(c, T, &F, &tiled);
  if (st) return st;
  // One row must fit the scratch: shrink the tile (tiles with exact halos
  // decode the same samples bit for bit) until it does.
  auto row_bytes = [&](int64_t f, bool t) {
    const int64_t ta = std::min<int64_t>(T, f + (t ? c->halo_l + c->halo_r : 0));
    return make_plan(c, 1, static_cast<int>(ta)).bytes;
  };
  if (row_bytes(F, tiled) > kScratchBytes) {
    if (row_bytes(1, true) > kScratchBytes)
      return fail(c, VOC_INVALID_PARAMS,
                  "one latent frame with its halos needs " + std::to_string(row_bytes(1, true)) +
                      " bytes of workspace, more than the " + std::to_string(kScratchBytes) +
                      "-byte no-allocation scratch");
    int64_t lo = 1, hi = F;  // row_bytes(lo) fits, row_bytes(hi) does not
    while (hi - lo > 1) {
      const int64_t mid = lo + (hi - lo) / 2;
      (row_bytes(mid, true) <= kScratchBytes ? lo : hi) = mid;
    }
    F = lo;
    tiled = true;
  }
  int64_t rows = 0;
  int T_alloc = 0;
  std::vector<int64_t> dst;
  std::vector<int> ints;
  st = decode_row_plan(c, B, T, F, tiled, &rows, &T_alloc, &dst, &ints);
  if (st) return st;
  // Rows per pass: as many as the scratch holds (passes run in stream order
  // on the same scratch).
  int64_t lo = 1, hi = rows + 1;  // lo rows fit, hi rows do not (or exceed the count)
  while (hi - lo > 1) {
    const int64_t mid = lo + (hi - lo) / 2;
    (make_plan(c, static_cast<int>(mid), T_alloc).bytes <= kScratchBytes ? lo : hi) = mid;
  }
  int64_t group = lo;
  if (c->cancel_fn) group = std::min(group, c->cancel_group);
  // No profiling events here (creating one may allocate).
  const bool prof = c->prof;
  c->prof = false;
  c->ws_override = c->scratch;
  c->ws_override_bytes = kScratchBytes;
  st = decode_rows(c, latent, T, rows, T_alloc, std::move(dst), std::move(ints), {5, B, T, rows}, pcm,
                   T * c->hop, static_cast<hipStream_t>(stream), group);
  c->ws_override = nullptr;
  c->ws_override_bytes = 0;
  c->prof = prof;
  return st;
}

VOC_API voc_status vocoder_encode(voc_ctx* c, const float* audio, int64_t B, int64_t T, float* latent,
                                  void* stream) {
  if (!c) return VOC_INVALID_PARAMS;
  const voc_config& g = c->cfg;
  if (g.enc_width[0] == 0) return fail(c, VOC_INVALID_PARAMS, "no encoder configured (enc_width)");
  if (!audio || !latent) return fail(c, VOC_INVALID_PARAMS, "NULL audio or latent");
  if ((reinterpret_cast<uintptr_t>(audio) | reinterpret_cast<uintptr_t>(latent)) & 15)
    return fail(c, VOC_INVALID_PARAMS, "audio and latent must be 16-byte aligned");
  if (B <= 0 || T <= 0 || B > 65535) return fail(c, VOC_INVALID_PARAMS, "B in [1, 65535] and T > 0 required");
  // The audio-rate layers read 64-byte rows per sample through the GEMM's
  // 32-bit buffer offsets: keep those planes below 4 GiB.
  if (T * c->hop > (int64_t(1) << 26) - (int64_t(1) << 16))
    return fail(c, VOC_INVALID_PARAMS, "T*hop exceeds 2^26 - 2^16 samples per row");
  if (!c->loaded) return fail(c, VOC_NOT_LOADED, "weights not loaded");
  if (cancel_requested(c)) return cancelled(c);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rows = static_cast<int>(B), nb = g.n_blocks, nr = g.n_res;
  const int* E = g.enc_width;
  const EncoderDev& en = c->W.enc;
  const Plan p = make_enc_plan(c, rows, static_cast<int>(T));
  voc_status st = ensure_ws(c, p.bytes);
  if (st) return st;
  const std::vector<int64_t> key = {4, B, T};
  if (c->rows_key != key) {
    std::vector<int64_t> dst(rows);
    std::vector<int> ints(5 * rows);
    for (int r = 0; r < rows; ++r) {
      ints[r] = static_cast<int>(T);                       // len (latent frames)
      ints[rows + r] = r;                                  // src_b
      ints[2 * rows + r] = 0;                              // start
      ints[3 * rows + r] = 0;                              // keep_lo
      ints[4 * rows + r] = static_cast<int>(T * c->hop);   // keep_hi
      dst[r] = r * T * c->hop;
    }
    st = upload_rows(c, p, std::move(dst), std::move(ints), s);
    if (st) return st;
    c->rows_key = key;
  }
  const Bufs Bf = bufs(c, p);
  const int* len = Bf.rows.len;
  int64_t t = T * c->hop;
  int rate = static_cast<int>(c->hop);
  const int op = c->op;
  st = launch(c, s, VOC_K_IMPORT, 0.0, static_cast<double>(rows) * t * (4 + kChunkBytes), "audio import launch",
              [&] { return launch_audio_import(op, audio, Bf.xlat, t, rows, s); });
  if (st) return st;
  // conv_in -> h and (unless the first unit takes it from h) its Snake1 operand.
  int cur = 0;
  float* hc = Bf.h;
  float* ho = Bf.h2;
  ConvIO io{};
  io.x = Bf.xlat;
  io.T_in = static_cast<int>(t);
  io.rate_in = rate;
  io.h_out = hc;
  if (!unit_xh(c, E[0])) {
    io.s_out = Bf.s[cur];
    io.snake_next = &en.blocks[0].units[0].a1;
  }
  st = run_conv(c, en.conv_in, io, rows, len, VOC_K_CONV_IN, s);
  if (st) return st;
  for (int b = 0; b < nb; ++b) {
    const EncBlockDev& eb = en.blocks[b];
    const bool xh = unit_xh(c, E[b]);
    for (int r = 0; r < nr; ++r) {
      // The last unit feeds the strided conv only through the block Snake.
      const bool keep_h = r + 1 < nr;
      const SnakeDev* next = keep_h ? (xh ? nullptr : &eb.units[r + 1].a1) : &eb.act;
      void* s_next = nullptr;
      st = run_res_unit(c, eb.units[r], xh ? nullptr : Bf.s[cur], Bf.s[cur ^ 1], Bf.u, hc, xh ? ho : nullptr,
                        next, &s_next, static_cast<int>(t), rate, rows, len, s, nullptr, keep_h);
      if (st) return st;
      if (s_next == Bf.s[cur ^ 1]) cur ^= 1;
      if (xh && keep_h) std::swap(hc, ho);
    }
    // Strided conv on Snake(h) -> the next block's h and first operand (the
    // last block: Snake_out of it, conv_out's operand).
    io = ConvIO{};
    io.x = Bf.s[cur];
    io.T_in = static_cast<int>(t);
    io.rate_in = rate;
    if (b + 1 < nb) {
      io.h_out = hc;
      if (!unit_xh(c, E[b + 1])) {
        io.s_out = Bf.s[cur ^ 1];
        io.snake_next = &en.blocks[b + 1].units[0].a1;
      }
    } else {
      io.s_out = Bf.s[cur ^ 1];
      io.snake_next = &en.out_act;
    }
    st = run_conv(c, eb.down, io, rows, len, VOC_K_ENC_DOWN, s);
    if (st) return st;
    if (io.s_out) cur ^= 1;
    t /= eb.down.down;
    rate /= eb.down.down;
  }
  // conv_out (k=3) -> its output as the projection's operand (no activation).
  io = ConvIO{};
  io.x = Bf.s[cur];
  io.T_in = static_cast<int>(t);
  io.rate_in = rate;
  io.s_out = Bf.u;
  st = run_conv(c, en.conv_out, io, rows, len, VOC_K_ENC_OUT, s);
  if (st) return st;
  io = ConvIO{};
  io.x = Bf.u;
  io.T_in = static_cast<int>(t);
  io.rate_in = rate;
  io.h_out = hc;
  st = run_conv(c, en.proj, io, rows, len, VOC_K_ENC_OUT, s);
  if (st) return st;
  const int C = g.latent_channels;
  return launch(c, s, VOC_K_EXPORT, 0.0, 8.0 * rows * C * T, "export launch",
                [&] { return launch_export(c->op, hc, latent, rows, C, static_cast<int>(T), s); });
}

namespace {
// The layers with carried context and their input layouts, in the order
// run_stack visits them: conv_in (k=7), per block the ConvTranspose1d (one
// input frame) and each unit's conv1 (6d frames of h when the unit computes
// its operand from h, else of the operand tensor), and the head (k=7 on h).
std::vector<voc_ctx::LayerState> stream_layers(const voc_ctx* c) {
  const voc_config& g = c->cfg;
  const int op_rows = 64 / op_size(c->op);  // channels per 64-byte operand row
  std::vector<voc_ctx::LayerState> v;
  const int h_rows = kHChunk * hsz(c);  // bytes per residual-stream frame row
  auto add = [&](int ctx, int64_t planes, int row_bytes) {
    voc_ctx::LayerState L;
    L.ctx = ctx;
    L.planes_per_row = planes;
    L.row_bytes = row_bytes;
    v.push_back(L);
  };
  // (Operand tensors of a two-term decoder hold twice the chunk planes; the
  // latent operand conv_in reads has one term.)
  add(6, (g.in_proj > 0 ? g.in_proj : g.latent_channels) / op_rows, kChunkBytes);
  for (int b = 0; b < g.n_blocks; ++b) {
    add(1, c->terms * g.width[b] / op_rows, kChunkBytes);
    const int C = g.width[b + 1];
    for (int r = 0; r < g.n_res; ++r)
      add(6 * g.dilation[r], unit_xh(c, C) ? C / 16 : c->terms * C / op_rows, unit_xh(c, C) ? h_rows : kChunkBytes);
  }
  // The head reads h (fp16, bf16 decoders) or Snake_out(h) in fp32.
  add(6, g.width[g.n_blocks] / 16, head_snake_at_load(c) ? h_rows : kChunkBytes);
  return v;
}
}  // namespace

VOC_API voc_status vocoder_stream_reset(voc_ctx* c, int64_t rows) {
  if (!c) return VOC_INVALID_PARAMS;
  if (!c->cfg.causal) return fail(c, VOC_INVALID_PARAMS, "streaming needs a causal configuration");
  if (c->cfg.tile_frames != 0) return fail(c, VOC_INVALID_PARAMS, "streaming needs tile_frames == 0");
  if (rows <= 0 || rows > 65535) return fail(c, VOC_INVALID_PARAMS, "rows must be in [1, 65535]");
  std::vector<voc_ctx::LayerState> L = stream_layers(c);
  size_t o = 0;
  int margin = 0;
  for (auto& l : L) {
    const size_t bytes = static_cast<size_t>(rows) * l.planes_per_row * l.ctx * l.row_bytes;
    l.off[0] = o;
    o = align_up(o + bytes);
    l.off[1] = o;
    o = align_up(o + bytes);
    margin = std::max(margin, l.ctx);
  }
  c->st_rows = 0;
  if (o > c->st_mem_bytes) {
    if (c->st_mem) {
      (void)hipDeviceSynchronize();
      (void)hipFree(c->st_mem);
      c->st_mem = nullptr;
      c->st_mem_bytes = 0;
    }
    hipError_t e = hipMalloc(&c->st_mem, o);
    if (e != hipSuccess) {
      c->st_mem = nullptr;
      return hip_fail(c, e, "stream state hipMalloc");
    }
    c->st_mem_bytes = o;
  }
  // Zero context: a new stream starts like the offline decode's zero left
  // padding.  (Synchronous: nothing of an earlier stream is in flight.)
  hipError_t e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemset(c->st_mem, 0, o);
  if (e != hipSuccess) return hip_fail(c, e, "stream state clear");
  c->st_layers = std::move(L);
  c->st_rows = rows;
  c->st_par = 0;
  c->st_margin = margin;
  return VOC_OK;
}

VOC_API voc_status vocoder_stream_decode(voc_ctx* c, const float* latent, int64_t t, float* pcm,
                                         void* stream) {
  if (!c) return VOC_INVALID_PARAMS;
  if (c->st_rows <= 0) return fail(c, VOC_INVALID_PARAMS, "vocoder_stream_reset has not been called");
  if (!latent || !pcm) return fail(c, VOC_INVALID_PARAMS, "NULL latent or pcm");
  if ((reinterpret_cast<uintptr_t>(latent) | reinterpret_cast<uintptr_t>(pcm)) & 15)
    return fail(c, VOC_INVALID_PARAMS, "latent and pcm must be 16-byte aligned");
  if (t <= 0 || t * c->hop + c->st_margin > (int64_t(1) << 31) - 1)
    return fail(c, VOC_INVALID_PARAMS, "t must be positive with t * hop below 2^31");
  if (t > row_frames_limit(c))
    return fail(c, VOC_INVALID_PARAMS, "t exceeds the frames the GEMMs can address (voc_config_max_frames)");
  if (!c->loaded) return fail(c, VOC_NOT_LOADED, "weights not loaded");
  if (cancel_requested(c)) return cancelled(c);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t rows = c->st_rows;
  const int mg = c->st_margin;
  const Plan p = make_plan(c, static_cast<int>(rows), static_cast<int>(t), mg);
  voc_status st = ensure_ws(c, p.bytes);
  if (st) return st;
  // Row r is stream r: the chunk's t frames, all of its samples kept.
  const std::vector<int64_t> key = {3, rows, t};
  if (c->rows_key != key) {
    std::vector<int64_t> dst(rows);
    std::vector<int> ints(5 * rows);
    for (int64_t r = 0; r < rows; ++r) {
      ints[r] = static_cast<int>(t);                          // len
      ints[rows + r] = static_cast<int>(r);                   // src_b
      ints[2 * rows + r] = 0;                                 // start
      ints[3 * rows + r] = 0;                                 // keep_lo
      ints[4 * rows + r] = static_cast<int>(t * c->hop);      // keep_hi
      dst[r] = r * c->cfg.out_channels * t * c->hop;
    }
    st = upload_rows(c, p, std::move(dst), std::move(ints), s);
    if (st) return st;
    c->rows_key = key;
  }
  const Bufs Bf = bufs(c, p);
  c->mg = mg;
  c->st_active = true;
  float* h_last = nullptr;
  st = run_import(c, latent, t, c->cfg.latent_channels, Bf.rows, static_cast<int>(rows),
                  static_cast<int>(t), Bf.xlat, nullptr, nullptr, s);
  if (!st) st = run_stack(c, Bf, static_cast<int>(rows), static_cast<int>(t), s, &h_last);
  if (!st)
    st = run_head(c, h_last, static_cast<int>(t * c->hop), Bf.rows, static_cast<int>(rows),
                  static_cast<int>(c->hop), pcm, t * c->hop, s, head_snake_at_load(c));
  c->mg = 0;
  c->st_active = false;
  if (st) return st;
  c->st_par ^= 1;
  return VOC_OK;
}

VOC_API int64_t vocoder_windows_output_length(const voc_ctx* c, int64_t n, int64_t L, int64_t L_last,
                                              int64_t cl, int64_t cr) {
  if (!c || !windows_valid(n, L, L_last, cl, cr)) return -1;
  int64_t kept = 0;
  for (int64_t k = 0; k < n; ++k) {
    int64_t lo, hi;
    window_keep(k, n, L, L_last, cl, cr, &lo, &hi);
    kept += hi - lo;
  }
  return kept * c->hop;
}

VOC_API voc_status vocoder_decode_windows(voc_ctx* c, const float* latents, int64_t n, int64_t sides,
                                          int64_t L, int64_t L_last, int64_t cl, int64_t cr, float* pcm,
                                          void* stream) {
  if (!c) return VOC_INVALID_PARAMS;
  if (!latents || !pcm) return fail(c, VOC_INVALID_PARAMS, "NULL latents or pcm");
  if ((reinterpret_cast<uintptr_t>(latents) | reinterpret_cast<uintptr_t>(pcm)) & 15)
    return fail(c, VOC_INVALID_PARAMS, "latents and pcm must be 16-byte aligned");
  if (sides != 1 && sides != 2) return fail(c, VOC_INVALID_PARAMS, "sides must be 1 or 2");
  if (!windows_valid(n, L, L_last, cl, cr))
    return fail(c, VOC_INVALID_PARAMS, "bad window count, lengths or crops (every window must keep a frame)");
  if (c->cfg.tile_frames != 0) return fail(c, VOC_INVALID_PARAMS, "windowed decode needs tile_frames == 0");
  if (L * c->hop > (int64_t(1) << 31) - 1) return fail(c, VOC_INVALID_PARAMS, "L*hop exceeds 2^31-1");
  if (L > row_frames_limit(c))
    return fail(c, VOC_INVALID_PARAMS, "L exceeds the frames the GEMMs can address (voc_config_max_frames)");
  const int64_t rows = n * sides;
  if (rows > 65535) return fail(c, VOC_INVALID_PARAMS, "too many rows (n_windows * sides > 65535)");
  if (!c->loaded) return fail(c, VOC_NOT_LOADED, "weights not loaded");
  const int64_t N = vocoder_windows_output_length(c, n, L, L_last, cl, cr);
  // Row k*sides + j decodes side j of window k (row k*sides + j of the
  // [n*sides, C, L] view) and writes the kept samples of its output channel
  // o at pcm[(j*O + o)*N + hop * (frames kept by windows 0..k-1)], O =
  // out_channels.
  std::vector<int64_t> dst(rows);
  std::vector<int> ints(5 * rows);
  int64_t before = 0;
  for (int64_t k = 0; k < n; ++k) {
    int64_t lo, hi;
    window_keep(k, n, L, L_last, cl, cr, &lo, &hi);
    for (int64_t j = 0; j < sides; ++j) {
      const int64_t r = k * sides + j;
      ints[r] = static_cast<int>(k == n - 1 ? L_last : L);        // len
      ints[rows + r] = static_cast<int>(r);                       // src_b
      ints[2 * rows + r] = 0;                                     // start
      ints[3 * rows + r] = static_cast<int>(lo * c->hop);         // keep_lo
      ints[4 * rows + r] = static_cast<int>(hi * c->hop);         // keep_hi
      dst[r] = j * c->cfg.out_channels * N + before * c->hop;
    }
    before += hi - lo;
  }
  const int64_t group = c->cancel_fn ? c->cancel_group * sides : rows;
  return decode_rows(c, latents, L, rows, static_cast<int>(L), std::move(dst), std::move(ints),
                     {1, n, sides, L, L_last, cl, cr}, pcm, N, static_cast<hipStream_t>(stream), group);
}

VOC_API voc_status vocoder_set_cancel(voc_ctx* c, voc_cancel_fn fn, void* user, int64_t group) {
  if (!c) return VOC_INVALID_PARAMS;
  if (group < 1) return fail(c, VOC_INVALID_PARAMS, "group must be at least 1");
  c->cancel_fn = fn;
  c->cancel_user = user;
  c->cancel_group = group;
  return VOC_OK;
}

VOC_API const char* vocoder_last_error(const voc_ctx* c) {
  return c ? c->err.c_str() : g_create_error.c_str();
}

VOC_API void vocoder_destroy(voc_ctx* c) {
  if (!c) return;
  (void)hipSetDevice(c->device);
  (void)hipDeviceSynchronize();
  free_weights(c->W);
  if (c->ws) (void)hipFree(c->ws);
  if (c->st_mem) (void)hipFree(c->st_mem);
  if (c->col_buf) (void)hipFree(c->col_buf);
  if (c->col_zero) (void)hipFree(c->col_zero);
  for (auto& r : c->pending) {
    (void)hipEventDestroy(r.e0);
    (void)hipEventDestroy(r.e1);
  }
  for (auto e : c->free_events) (void)hipEventDestroy(e);
  delete c;
}

VOC_API voc_status vocoder_profile_enable(voc_ctx* c, int enable) {
  if (!c) return VOC_INVALID_PARAMS;
  c->prof = enable != 0;
  return VOC_OK;
}

VOC_API voc_status vocoder_profile_select(voc_ctx* c, uint32_t kinds) {
  if (!c || (kinds >> VOC_K_COUNT) != 0) return VOC_INVALID_PARAMS;
  c->prof_kinds = kinds;
  return VOC_OK;
}

VOC_API voc_status vocoder_profile_reset(voc_ctx* c) {
  if (!c) return VOC_INVALID_PARAMS;
  voc_status st = finalize_profile(c);
  for (auto& s : c->stats) s = voc_profile_stat{};
  return st;
}

VOC_API voc_status vocoder_profile_read(voc_ctx* c, int kind, voc_profile_stat* out) {
  if (!c || !out || kind < 0 || kind >= VOC_K_COUNT) return VOC_INVALID_PARAMS;
  voc_status st = finalize_profile(c);
  if (st) return st;
  *out = c->stats[kind];
  return VOC_OK;
}

// ------------------------------------------------------------------ debug

namespace {
struct StageInfo {
  int kind;  // 0 conv_in, 1 convT, 2 res unit, 3 head
  int b, r;
  int c_in, c_out, ups;
};
bool stage_info(const voc_ctx* c, int k, StageInfo* si) {
  const voc_config& g = c->cfg;
  const int n = 2 + g.n_blocks * (1 + g.n_res);
  if (k < 0 || k >= n) return false;
  if (k == 0) {
    *si = {0, 0, 0, g.latent_channels, g.width[0], 1};
    return true;
  }
  if (k == n - 1) {
    *si = {3, 0, 0, g.width[g.n_blocks], g.out_channels, 1};
    return true;
  }
  const int b = (k - 1) / (1 + g.n_res), j = (k - 1) % (1 + g.n_res);
  if (j == 0)
    *si = {1, b, 0, g.width[b], g.width[b + 1], g.stride[b]};
  else
    *si = {2, b, j - 1, g.width[b + 1], g.width[b + 1], 1};
  return true;
}
}  // namespace

VOC_API int voc_dbg_stage_count(const voc_ctx* c) {
  return c ? 2 + c->cfg.n_blocks * (1 + c->cfg.n_res) : VOC_INVALID_PARAMS;
}

VOC_API voc_status voc_dbg_stage_shape(const voc_ctx* c, int stage, int64_t T_in, int64_t* c_in,
                                       int64_t* c_out, int64_t* t_out) {
  StageInfo si;
  if (!c || !c_in || !c_out || !t_out || !stage_info(c, stage, &si)) return VOC_INVALID_PARAMS;
  *c_in = si.c_in;
  *c_out = si.c_out;
  *t_out = T_in * si.ups;
  return VOC_OK;
}

VOC_API voc_status voc_dbg_run_stage(voc_ctx* c, int stage, const float* in, int64_t B, int64_t T_in,
                                     float* out, void* stream) {
  if (!c) return VOC_INVALID_PARAMS;
  StageInfo si;
  if (!stage_info(c, stage, &si)) return fail(c, VOC_INVALID_PARAMS, "bad stage index");
  if (!in || !out || B <= 0 || T_in <= 0 || B > 65535) return fail(c, VOC_INVALID_PARAMS, "bad stage arguments");
  if ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(c, VOC_INVALID_PARAMS, "buffers must be 16-byte aligned");
  if (!c->loaded) return fail(c, VOC_NOT_LOADED, "weights not loaded");
  if (c->terms == 2)
    return fail(c, VOC_INVALID_PARAMS, "the stage runner serves one-term decoders (operand_terms 0 or 1)");
  const int64_t t_out = T_in * si.ups;
  if (t_out > (int64_t(1) << 31) - 1) return fail(c, VOC_INVALID_PARAMS, "T too large");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int rows = static_cast<int>(B);
  // Workspace: enough for the stage's input and output at these frames; the
  // row metadata treats each row as a whole clip of T_in frames at rate 1.
  int64_t cmax = std::max(si.c_in, si.c_out);
  if (si.kind == 0) cmax = std::max<int64_t>(cmax, c->cfg.in_proj);  // dec_in_proj output in u
  const size_t es = op_size(c->op);
  const size_t act_in = static_cast<size_t>(rows) * si.c_in * T_in;
  const size_t act_out = static_cast<size_t>(rows) * cmax * t_out;
  size_t o = 0;
  const size_t off_h = o; o = align_up(o + 4 * std::max(act_in, act_out));
  const bool xh = si.kind == 2 && unit_xh(c, static_cast<int>(si.c_out));
  const bool af = c->cfg.af_snake != 0 || c->split_snake;  // every Snake a launch of its own
  const size_t off_h2 = o; if (xh || af) o = align_up(o + 4 * std::max(act_in, act_out));
  const size_t off_s0 = o; o = align_up(o + es * act_in);
  const size_t off_s1 = o; o = align_up(o + es * act_out);
  const size_t off_u = o; o = align_up(o + es * act_out);
  const size_t off_meta = o; o = align_up(o + rows * (5 * sizeof(int) + sizeof(int64_t)) + 64);
  voc_status st = ensure_ws(c, o);
  if (st) return st;
  char* base = static_cast<char*>(c->ws);
  float* h = reinterpret_cast<float*>(base + off_h);
  float* h2 = reinterpret_cast<float*>(base + off_h2);
  void* s0 = base + off_s0;
  void* s1 = base + off_s1;
  void* u = base + off_u;
  Plan p{};
  p.rows = rows;
  p.off_meta = off_meta;
  std::vector<int64_t> dst(rows);
  std::vector<int> ints(5 * rows);
  for (int r = 0; r < rows; ++r) {
    ints[r] = static_cast<int>(T_in);
    ints[rows + r] = r;
    ints[2 * rows + r] = 0;
    ints[3 * rows + r] = 0;
    ints[4 * rows + r] = static_cast<int>(T_in);
    dst[r] = static_cast<int64_t>(r) * c->cfg.out_channels * T_in;
  }
  st = upload_rows(c, p, std::move(dst), std::move(ints), s);
  if (st) return st;
  c->rows_key.clear();  // the decode's cached metadata is gone
  char* m = base + off_meta;
  RowInfo ri{};
  ri.dst = reinterpret_cast<const int64_t*>(m);
  const int* ib = reinterpret_cast<const int*>(m + sizeof(int64_t) * rows);
  ri.len = ib;
  ri.src_b = ib + rows;
  ri.start = ib + 2 * rows;
  ri.keep_lo = ib + 3 * rows;
  ri.keep_hi = ib + 4 * rows;
  const Weights& W = c->W;
  const int T = static_cast<int>(T_in);
  ConvIO io{};
  switch (si.kind) {
    case 0:
      st = run_import(c, in, T_in, si.c_in, ri, rows, T, s0, nullptr, nullptr, s);
      if (st) return st;
      io.x = s0; io.T_in = T; io.rate_in = 1;
      if (W.in_proj.cout > 0) {
        io.s_out = u;
        st = run_conv(c, W.in_proj, io, rows, ri.len, VOC_K_IN_PROJ, s);
        if (st) return st;
        io = ConvIO{};
        io.x = u; io.T_in = T; io.rate_in = 1;
      }
      io.h_out = h;
      st = run_conv(c, W.conv_in, io, rows, ri.len, VOC_K_CONV_IN, s);
      break;
    case 1:
      if (af) {  // import h, then its alias-free Snake into the operand
        st = run_import(c, in, T_in, si.c_in, ri, rows, T, nullptr, nullptr, h, s);
        if (!st) st = run_af(c, W.blocks[si.b].act, h, si.c_in, T, 1, rows, ri.len, s0, c->op, s);
      } else {
        st = run_import(c, in, T_in, si.c_in, ri, rows, T, s0, &W.blocks[si.b].act, nullptr, s);
      }
      if (st) return st;
      io.x = s0; io.T_in = T; io.rate_in = 1; io.h_out = h;
      st = run_convt(c, W.blocks[si.b].ct, io, rows, ri.len, s);
      break;
    case 2: {
      // The same kernel path as in a decode: with the operand computed from
      // h, the import writes h only and the unit writes h2.
      const UnitDev& un = W.blocks[si.b].units[si.r];
      if (af) {
        st = run_import(c, in, T_in, si.c_in, ri, rows, T, nullptr, nullptr, h, s);
        if (!st) st = run_res_unit_af(c, un, h, h2, s0, u, T, 1, rows, ri.len, s);
        break;
      }
      st = run_import(c, in, T_in, si.c_in, ri, rows, T, xh ? nullptr : s0, &un.a1, h, s);
      if (st) return st;
      st = run_res_unit(c, un, s0, s1, u, h, xh ? h2 : nullptr, nullptr, nullptr, T, 1, rows, ri.len, s);
      if (xh) h = h2;
      break;
    }
    default:
      if (af) {  // the head reads AF(h), computed into h2
        st = run_import(c, in, T_in, si.c_in, ri, rows, T, nullptr, nullptr, h, s);
        if (!st) st = run_af(c, W.head_act, h, si.c_in, T, 1, rows, ri.len, h2, OP_F32, s);
        if (st) return st;
        return run_head(c, h2, T, ri, rows, 1, out, T_in, s);
      }
      if (const SnakeDev* hs = head_snake_at_load(c)) {  // the head applies Snake_out to h
        st = run_import(c, in, T_in, si.c_in, ri, rows, T, nullptr, nullptr, h, s);
        if (st) return st;
        return run_head(c, h, T, ri, rows, 1, out, T_in, s, hs);
      }
      st = run_import(c, in, T_in, si.c_in, ri, rows, T, nullptr, nullptr, h, s, &W.head_act);
      if (st) return st;
      return run_head(c, h, T, ri, rows, 1, out, T_in, s);
  }
  if (st) return st;
  return launch(c, s, VOC_K_EXPORT, 0.0, 8.0 * rows * si.c_out * t_out, "export launch",
                [&] { return launch_export(c->op, h, out, rows, si.c_out, static_cast<int>(t_out), s); });
}

VOC_API voc_status voc_dbg_peak(int what, int64_t n, double* value, void* stream) {
  if (!value || n <= 0 || what < 0 || what > 4) return VOC_INVALID_PARAMS;
  if (what == 0 && (n & 15)) return VOC_INVALID_PARAMS;
  *value = 0.0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* b0 = nullptr;
  void* b1 = nullptr;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  voc_status st = VOC_DEVICE_ERROR;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (what == 0) {  // HBM: a plain copy of n bytes; reads + writes counted
    if (e == hipSuccess) e = hipMalloc(&b0, static_cast<size_t>(n));
    if (e == hipSuccess) e = hipMalloc(&b1, static_cast<size_t>(n));
    if (e == hipSuccess) e = hipMemsetAsync(b0, 1, static_cast<size_t>(n), s);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) e = launch_copy(b1, b0, n, s);
    const int reps = 5;
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    for (int i = 0; i < reps && e == hipSuccess; ++i) e = launch_copy(b1, b0, n, s);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && ms > 0.f) {
      *value = 2.0 * reps * static_cast<double>(n) / (ms * 1e-3) / 1e9;
      st = VOC_OK;
    }
  } else {  // matrix cores: n iterations of an MFMA loop, fp32 (1, 3) or bf16 (2, 4), 16x16 or 32x32
    const int op = what == 1 || what == 3 ? OP_F32 : OP_BF16;
    const bool wide = what >= 3;
    auto loop = [&](int64_t it) {
      return wide ? launch_mfma32_loop(op, it, static_cast<float*>(b0), s)
                  : launch_mfma_loop(op, it, static_cast<float*>(b0), s);
    };
    if (e == hipSuccess) e = hipMalloc(&b0, static_cast<size_t>(mfma_loop_blocks()) * 256 * sizeof(float));
    if (e == hipSuccess) e = loop(std::max<int64_t>(1, n / 10));
    if (e == hipSuccess) e = hipEventRecord(e0, s);
    if (e == hipSuccess) e = loop(n);
    if (e == hipSuccess) e = hipEventRecord(e1, s);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e == hipSuccess && ms > 0.f) {
      *value = (wide ? mfma32_loop_flops(op, n) : mfma_loop_flops(op, n)) / (ms * 1e-3) / 1e12;
      st = VOC_OK;
    }
  }
  (void)hipStreamSynchronize(s);
  if (b0) (void)hipFree(b0);
  if (b1) (void)hipFree(b1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return st;
}

VOC_API voc_status voc_dbg_copy(void* dst, const void* src, int64_t bytes, void* stream) {
  if (!dst || !src || bytes <= 0 || (bytes & 15) ||
      ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) & 15))
    return VOC_INVALID_PARAMS;
  hipError_t e = launch_copy(dst, src, bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? VOC_OK : VOC_DEVICE_ERROR;
}
