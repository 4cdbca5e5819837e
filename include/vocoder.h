/*
 * vocoder.h -- C ABI of the MI355X DAC-style waveform decoder (libvocoder.so).
 *
 * Plain C99, no C++ or PyTorch types.  Every entry point returns a voc_status
 * (0 = success, negative = error) unless stated otherwise, never throws, and
 * records a human-readable message retrievable with vocoder_last_error().
 *
 * The decoder (minimaxmusic.cpp ARCHITECTURE page, section "Flow VAE"; the
 * DAC stack of the qwentts.cpp ARCHITECTURE page, "Audio tokenizer decoder"):
 *
 *   x   = dec_in_proj(latent)                   optional Conv1d k=1, bias, no weight norm
 *   h   = conv_in(x)                            Conv1d k=7, zero "same" padding, bias
 *   per block b with stride s:
 *     h = conv_t1(Snake(h))                     ConvTranspose1d k=2s, stride s, crop ceil(s/2)
 *   (causal configurations: every k=7 conv pads (K-1)*d on the left only and
 *    the ConvTranspose1d keeps full[0, T*s), qwentts.cpp ARCHITECTURE, "Audio
 *    tokenizer decoder" and "Streaming decode (stateful path)")
 *     per residual unit with dilation d (1, 3, 9):
 *       h = h + conv2(Snake2(conv1_d(Snake1(h))))   conv1 k=7 dilation d, conv2 k=1
 *   pcm = tanh(conv_out(Snake(h)))              Conv1d k=7 to out_channels (1 or 2), bias
 *
 *   Snake(x)     = x + sin^2(alpha x) / (alpha + 1e-9)   alpha read verbatim
 *   SnakeBeta(x) = x + sin^2(alpha x) / (beta  + 1e-9)
 *
 * Alias-free configurations (af_snake = 1; the H3 audio VAE of the
 * TensorSharp minimax-h3 page: every nonlinearity inside a 2x upsample /
 * activate / 2x downsample sandwich) replace every Snake above by
 *   AF(x) = down2(Snake(up2(x)))
 * with one 12-tap Kaiser-windowed sinc low-pass f (cutoff a quarter of the
 * 2x rate, transition half-width 0.3 of its sample rate, unit DC gain):
 *   up2:   replicate-pad 5 frames, zero-stuff, filter with 2f, keep the 2T
 *          samples aligned with x (u[n] sits at time n/2 - 1/4);
 *   down2: replicate-pad 5 / 6 samples, filter with f, keep every second.
 * Each AF output frame depends on input frames t-5 .. t+5.
 *
 * Weight norm is folded once at load: w = g * v / ||v||, the norm taken over
 * each slice along axis 0 of the stored tensor (minimaxmusic.cpp ARCHITECTURE,
 * "Models").
 *
 * Stereo: the 128 latent channels of a stereo track are two independent
 * 64-channel tracks, channels 0..63 left (minimaxmusic.cpp ARCHITECTURE,
 * "Flow VAE").  A caller holding [b, 128, t] passes the view [2b, 64, t]
 * (rows 2i = left, 2i+1 = right) and reads the [2b, 1, N] output as [b, 2, N].
 * vocoder_decode_windows does the same fold per window and writes planar
 * stereo.
 *
 * Conventions follow the qwentts.cpp public ABI (ARCHITECTURE page, "Public
 * API" and "ABI guarantee"): an opaque context, a parameter struct carrying
 * abi_version, a status enum, a last-error string, extern "C" with only these
 * symbols exported.
 *
 * Threading: one context per host thread / stream.  A context is not safe for
 * concurrent calls.
 */
#ifndef VOCODER_H
#define VOCODER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define VOC_ABI_VERSION 4
#define VOC_MAX_BLOCKS 8
#define VOC_MAX_RES 4
/* Bytes of the device array vocoder_decode_noalloc uses as its workspace
 * (one copy per GPU the library runs on, held until the process ends). */
#define VOC_NOALLOC_SCRATCH_BYTES 268435456

typedef struct voc_ctx voc_ctx;

typedef enum voc_status {
  VOC_OK = 0,
  VOC_INVALID_PARAMS = -1, /* bad config, shape, pointer or size            */
  VOC_BAD_WEIGHTS = -2,    /* missing/unknown/mis-shaped tensor, ||v|| = 0,  */
                           /* or a non-finite value                          */
  VOC_OOM = -3,            /* device allocation failed or exceeds the cap    */
  VOC_DEVICE_ERROR = -4,   /* a HIP call or kernel launch failed             */
  VOC_NOT_LOADED = -5,     /* decode before a successful load_weights        */
  VOC_CANCELLED = -6       /* the cancel hook asked to stop (vocoder_set_cancel) */
} voc_status;

typedef enum voc_dtype {
  VOC_F32 = 0,  /* fp32 weights and matrix-core operands, fp32 accumulate   */
  VOC_BF16 = 1  /* bf16 weights (cast after the fold) and bf16 operands,    */
                /* fp32 accumulate and epilogues, fp16 residual stream       */
                /* (operand_terms = 2: two bf16 terms per operand, below)    */
} voc_dtype;

typedef enum voc_act { VOC_SNAKE = 0, VOC_SNAKE_BETA = 1 } voc_act;

/*
 * Architecture description.  Constraints (checked by voc_config_validate):
 * abi_version == VOC_ABI_VERSION; 1 <= n_blocks <= VOC_MAX_BLOCKS;
 * 1 <= n_res <= VOC_MAX_RES; 1 <= dilation[r] <= 9; stride[b] >= 1;
 * in_kernel == res_kernel == out_kernel == 7; widths, latent_channels and a
 * non-zero in_proj positive multiples of 16 (F32) or 32 (BF16), at most 8192,
 * width[n_blocks] <= 512; convt_crop == 0, or 1 with causal == 1;
 * tile_frames >= 0; in_proj >= 0;
 * causal is 0 or 1; an encoder (enc_width[0] > 0) needs every enc_width[b]
 * (b <= n_blocks) a positive multiple of 16 (F32) or 32 (BF16), at most
 * 8192, even strides and causal == 0; af_snake is 0 or 1, and 1 needs
 * causal == 0 and no encoder; out_channels is 1 or 2; operand_terms is 0, 1
 * or 2, and 2 needs dtype == VOC_BF16, af_snake == 0, in_proj == 0 and no
 * encoder.
 */
typedef struct voc_config {
  int abi_version;
  int latent_channels;             /* C of the latent                          */
  int n_blocks;                    /* upsampling blocks                         */
  int width[VOC_MAX_BLOCKS + 1];   /* width[0] = conv_in output, width[b+1] =   */
                                   /* block b output                            */
  int stride[VOC_MAX_BLOCKS];      /* block strides; ConvTranspose1d k = 2*s    */
  int in_kernel, res_kernel, out_kernel;
  int n_res;                       /* residual units per block                  */
  int dilation[VOC_MAX_RES];       /* their conv1 dilations                     */
  int act;                         /* voc_act                                   */
  int dtype;                       /* voc_dtype                                 */
  int snake_log_params;            /* 0: alpha/beta used as given; 1: the       */
                                   /* stored values are logs, exp() at load     */
  int convt_crop;                  /* 0: the crop that goes with `causal`:      */
                                   /* keep full[n + ceil(s/2)], n < T*s, or     */
                                   /* full[0, T*s) for a causal decoder; 1: the */
                                   /* causal crop, named explicitly (accepted   */
                                   /* with causal = 1 only: the pages pair the  */
                                   /* causal crop with causal convs)            */
  int tile_frames;                 /* 0: decode whole rows; F > 0: decode time  */
                                   /* tiles of F latent frames with exact halos */
  int in_proj;                     /* 0: none; P > 0: dec_in_proj, a Conv1d k=1 */
                                   /* latent_channels -> P with bias and no     */
                                   /* weight norm, ahead of conv_in (which then */
                                   /* has P input channels): the DAV decoder    */
                                   /* of minimaxmusic.cpp ARCHITECTURE, "Flow   */
                                   /* VAE" (64 -> 1024, conv_in 1024 -> 1536)   */
  int causal;                      /* 0: "same" padding and centered crop; 1:   */
                                   /* causal k=7 convs (left pad (K-1)*d) and   */
                                   /* ConvTranspose1d keeping full[0, T*s)      */
  int enc_width[VOC_MAX_BLOCKS + 1]; /* encoder widths (all 0: no encoder):     */
                                   /* conv_in 1 -> enc_width[0], block b        */
                                   /* enc_width[b] -> enc_width[b+1] with the   */
                                   /* decoder's strides in reverse order        */
  int af_snake;                    /* 0: plain Snake; 1: every Snake alias-free */
                                   /* (the 2x up / Snake / 2x down sandwich     */
                                   /* described above)                          */
  int out_channels;                /* conv_out output channels: 1 (mono rows)   */
                                   /* or 2 (one row decodes to stereo; the H3   */
                                   /* audio VAE, 32 channels -> stereo 32 kHz)  */
  int operand_terms;               /* 0 or 1: each matrix-core activation       */
                                   /* operand is one bf16 value; 2 (BF16): two  */
                                   /* bf16 terms hi = bf16(x), lo = bf16(x-hi), */
                                   /* both multiplied by the same bf16 weights  */
                                   /* with fp32 accumulation: the operand holds */
                                   /* x to ~2^-17 of its size, for twice the    */
                                   /* matrix work and operand bytes (the bf16   */
                                   /* weights and latent are unchanged)         */
} voc_config;

/* Fill *cfg with the full-width stereo window decoder: latent 64, widths
 * 1024/512/256/128/64, strides 8,8,4,2, dilations 1,3,9, Snake, F32, untiled,
 * no dec_in_proj, plain Snake, one output channel. */
void voc_config_default(voc_config *cfg);

/* Host-only checks of *cfg (no device is touched). */
voc_status voc_config_validate(const voc_config *cfg);

/* Samples per latent frame (product of the strides), or a negative status. */
int64_t voc_config_hop(const voc_config *cfg);

/* Exact receptive-field halo H in latent frames (host-only): decoding latent
 * frames [t0-H, t1+H) (clamped to the clip) reproduces the untiled output on
 * samples [t0*hop, t1*hop).  For causal configurations H is the left halo
 * and no frames to the right are needed.  Negative status if *cfg is invalid. */
int voc_config_halo(const voc_config *cfg);

/* Largest latent frames per decoded row that the matrix-core kernels can
 * address (host-only): a whole row of an untiled decode, a window of
 * vocoder_decode_windows, a stream chunk, or a time tile plus its two halos.
 * The GEMMs read each activation channel plane (64 bytes per frame) through
 * buffer loads with 32-bit byte offsets, so a plane must stay below 4 GiB;
 * the bound is set by the highest-rate layer that runs as a GEMM (for the
 * default decoder the last ConvTranspose1d, at hop/2 frames per latent
 * frame: 262 k latent frames, about 50 min of 44.1 kHz audio).
 * vocoder_decode splits longer untiled rows into time tiles on its own.
 * Negative status if *cfg is invalid. */
int64_t voc_config_max_frames(const voc_config *cfg);

/* Create a context on HIP device hip_device.  Validates *cfg first (no device
 * call happens if it is invalid).  *out receives the context or NULL. */
voc_status vocoder_create(const voc_config *cfg, int hip_device, voc_ctx **out);

/*
 * One named host tensor, fp32, contiguous, caller-owned.  Names and shapes
 * (PyTorch conventions; size-1 dims may be dropped, e.g. g as [d0] or
 * [d0,1,1], alpha as [C] or [1,C,1]):
 *   dec_in_proj.{weight [P,Clat,1], bias [P]}      (only with in_proj = P > 0)
 *   conv_in.{weight_v [W0,Cin,7], weight_g [W0,1,1], bias [W0]}
 *                                     (Cin = in_proj if non-zero, else Clat)
 *   blocks.{b}.snake1.alpha [1,Wb,1]          (+ .beta for SnakeBeta)
 *   blocks.{b}.conv_t1.{weight_v [Wb,Wb+1,2s], weight_g [Wb,1,1], bias [Wb+1]}
 *   blocks.{b}.res_units.{r}.snake1.alpha, .conv1.{weight_v [W,W,7], weight_g, bias},
 *                           .snake2.alpha, .conv2.{weight_v [W,W,1], weight_g, bias}
 *   snake_out.alpha [1,Wn,1];  conv_out.{weight_v [O,Wn,7], weight_g [O,1,1], bias [O]}
 *                                     (O = out_channels)
 * and with an encoder (E = enc_width, s_b = stride[n_blocks-1-b]):
 *   encoder.conv_in.{weight_v [E0,1,7], weight_g, bias}
 *   encoder.blocks.{b}.res_units.{r}.{snake1, conv1 [Eb,Eb,7], snake2, conv2 [Eb,Eb,1]}
 *   encoder.blocks.{b}.snake.alpha [1,Eb,1]; encoder.blocks.{b}.down.{weight_v [Eb+1,Eb,2s_b], ...}
 *   encoder.snake_out.alpha [1,En,1]; encoder.conv_out.{weight_v [En,En,3], ...}
 *   encoder.proj.{weight_v [Clat,En,1], weight_g, bias}
 */
typedef struct voc_tensor {
  const char *name;
  const float *data;
  int ndim;
  int64_t shape[4];
} voc_tensor;

/*
 * Copy the n tensors to the device, fold weight norm there (fp64 norms),
 * cast (BF16 configs: fp64 -> fp32 -> bf16, round to nearest even), precompute
 * 1/(alpha+1e-9) or 1/(beta+1e-9), and repack into the kernels' layouts.
 * All-or-nothing: on any error the previously loaded weights (if any) stay
 * in place.  Synchronizes the device.  Errors: VOC_BAD_WEIGHTS (missing,
 * duplicate, unknown or mis-shaped tensor; ||v|| = 0; non-finite value),
 * VOC_INVALID_PARAMS (NULL pointers), VOC_OOM, VOC_DEVICE_ERROR.
 */
voc_status vocoder_load_weights(voc_ctx *ctx, const voc_tensor *tensors, int n);

/* Output samples per row for T latent frames (T * hop), or -1 on bad input. */
int64_t vocoder_output_length(const voc_ctx *ctx, int64_t T);

/*
 * Decode latent (device, fp32, [B, latent_channels, T] contiguous) into pcm
 * (device, fp32, [B, out_channels, T*hop] contiguous) on hip_stream (a hipStream_t;
 * NULL = the null stream).  Asynchronous: enqueues kernels and returns; no
 * host synchronization except when the library-owned workspace has to grow
 * (hipMalloc), the first time a larger B*T is seen.  Both buffers stay owned
 * by the caller and must be 16-byte aligned.  BF16 configs round the latent
 * to bf16 as a matrix-core operand.  With tile_frames > 0 the rows are cut
 * into tiles of tile_frames latent frames plus the exact halo on each side
 * and all tiles are decoded as one batch.
 * Untiled rows longer than voc_config_max_frames() are decoded in time
 * tiles with exact halos as well (the same samples, bit for bit).
 * Errors: VOC_INVALID_PARAMS (NULL/misaligned pointers, B or T <= 0, T*hop
 * beyond 2^31 - 1 samples per row, a tile plus halos beyond
 * voc_config_max_frames(), more than 65535 rows of tiles),
 * VOC_NOT_LOADED, VOC_OOM, VOC_DEVICE_ERROR, VOC_CANCELLED.
 */
voc_status vocoder_decode(voc_ctx *ctx, const float *latent, int64_t B, int64_t T,
                          float *pcm, void *hip_stream);

/*
 * vocoder_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same arguments, checks and output, bit for bit, but no hipMalloc,
 * hipFree or other allocating call.  The workspace is a fixed device array
 * of VOC_NOALLOC_SCRATCH_BYTES (256 MiB) per GPU inside the library: rows
 * (time tiles with exact halos when one whole row does not fit, the same
 * samples bit for bit) are decoded in passes of as many rows as it holds,
 * in stream order.  Nothing in it needs clearing between calls: every
 * kernel reads only what the same call has written (the convolutions' zero
 * padding comes from bounds, not memory).  Every context and stream on one
 * GPU shares that GPU's array, so calls that overlap on one GPU (different
 * streams, or host threads) race and must be serialized by the caller.  The
 * row metadata is copied from host memory with hipMemcpyAsync; profiling
 * events are not recorded.  Same cancel hook behaviour as vocoder_decode.
 * Errors: those of vocoder_decode, and VOC_INVALID_PARAMS when one latent
 * frame with its halos needs more workspace than the array holds (a message
 * gives the size), VOC_DEVICE_ERROR when the array is unavailable.
 */
voc_status vocoder_decode_noalloc(voc_ctx *ctx, const float *latent, int64_t B, int64_t T,
                                  float *pcm, void *hip_stream);

/*
 * Windowed decode with stitching (minimaxmusic.cpp ARCHITECTURE, "Inference
 * recipe", "Decode and stitch" and "Post-processing"): each latent window is
 * decoded on its own; every window but the first drops crop_left latent
 * frames (x hop samples) on the left, every window but the last drops
 * crop_right frames on the right, and the kept segments are concatenated in
 * window order, clamped to [-1, 1] (the identity after tanh), into planar
 * output.  With the pages' windows of 689 frames and crops 86 / 258, windows
 * that start 689 - 86 - 258 = 345 frames apart tile the track seamlessly.
 *
 * latents: device fp32 [n_windows, sides * latent_channels, L] contiguous;
 *   side j of window k is channels [j*C, (j+1)*C) (stereo: 0..63 left), so
 *   the array is the [n_windows * sides, C, L] rows that vocoder_decode takes.
 *   The last window holds L_last valid frames (1 <= L_last <= L); its frames
 *   at and beyond L_last are ignored.
 * pcm: device fp32 [sides * out_channels, N] planar ([L: N][R: N] for
 *   stereo; output channel o of side j is plane j * out_channels + o) with
 *   N = vocoder_windows_output_length(...) samples per plane.
 * sides is 1 (mono) or 2 (stereo).  Every window must keep at least one
 * frame (e.g. L > crop_left + crop_right for the middle windows).  Requires
 * tile_frames == 0.  Same asynchrony and buffer ownership as vocoder_decode;
 * one batched decode of all n_windows * sides rows.
 * Errors: VOC_INVALID_PARAMS (NULL/misaligned pointers, bad counts or crops,
 * a window keeping nothing, tile_frames != 0, L beyond
 * voc_config_max_frames()), VOC_NOT_LOADED, VOC_OOM, VOC_DEVICE_ERROR,
 * VOC_CANCELLED.
 */
voc_status vocoder_decode_windows(voc_ctx *ctx, const float *latents, int64_t n_windows,
                                  int64_t sides, int64_t L, int64_t L_last,
                                  int64_t crop_left, int64_t crop_right, float *pcm,
                                  void *hip_stream);

/*
 * Streaming decode (causal configurations; qwentts.cpp ARCHITECTURE,
 * "Streaming decode (stateful path)"): `rows` independent streams decoded
 * chunk by chunk, each chunk's output equal bit for bit to the matching
 * samples of the offline decode of everything the stream has received.
 *
 * vocoder_stream_reset(ctx, rows) starts `rows` streams with empty history
 * (the next chunk decodes as the start of a clip: zero left padding).
 * vocoder_stream_decode decodes the next t >= 1 latent frames of every
 * stream, latent: device fp32 [rows, latent_channels, t] contiguous, into
 * pcm: device fp32 [rows, out_channels, t*hop] contiguous.  Each layer with context
 * carries its last input frames from chunk to chunk ((K-1)*d frames for a
 * causal k=7 conv, one input frame for a ConvTranspose1d, whose polyphase
 * form needs x[n-1] where the pages carry the col2im tail), so every chunk
 * decodes only its own frames.  Same asynchrony and ownership as
 * vocoder_decode; the state lives in library memory (hipMalloc at reset,
 * cleared to zero there, which is the offline decode's zero left padding).
 * Errors: VOC_INVALID_PARAMS (non-causal or tiled configuration, rows or t
 * out of range (t at most voc_config_max_frames()), NULL/misaligned
 * pointers, decode before reset), VOC_NOT_LOADED, VOC_OOM, VOC_DEVICE_ERROR,
 * VOC_CANCELLED (before the chunk: the stream state is unchanged).
 */
voc_status vocoder_stream_reset(voc_ctx *ctx, int64_t rows);
voc_status vocoder_stream_decode(voc_ctx *ctx, const float *latent, int64_t t, float *pcm,
                                 void *hip_stream);

/*
 * Encode (minimaxmusic.cpp ARCHITECTURE, "Flow VAE": the encoder mirrors the
 * decoder; its output is the posterior mean, no sampling): audio (device,
 * fp32, [B, 1, T*hop] contiguous, one mono row per side) -> latent (device,
 * fp32, [B, latent_channels, T] contiguous).  Per row: conv_in (k=7), per
 * block three residual units, Snake and a strided Conv1d (k = 2s, stride s,
 * pad s/2), then Snake, conv_out (k=3) and the projection (k=1).  Same
 * asynchrony and ownership as vocoder_decode.  BF16 configs round the audio
 * to bf16 as a matrix-core operand.
 * Errors: VOC_INVALID_PARAMS (no encoder configured, NULL/misaligned
 * pointers, B or T <= 0, T*hop beyond 2^26 - 2^16 samples per row, which
 * keeps the audio-rate layers' planes below 4 GiB), VOC_NOT_LOADED, VOC_OOM,
 * VOC_DEVICE_ERROR, VOC_CANCELLED.
 */
voc_status vocoder_encode(voc_ctx *ctx, const float *audio, int64_t B, int64_t T, float *latent,
                          void *hip_stream);

/* Samples per side that vocoder_decode_windows writes for these arguments:
 * hop times the kept latent frames of all windows; -1 if they are invalid. */
int64_t vocoder_windows_output_length(const voc_ctx *ctx, int64_t n_windows, int64_t L,
                                      int64_t L_last, int64_t crop_left, int64_t crop_right);

/*
 * Cancellation (minimaxmusic.cpp ARCHITECTURE, "mm-server reference",
 * "Concurrency": a job's cancel flag is polled between VAE windows;
 * qwentts.cpp ARCHITECTURE, "Public API": a polled cancel returns a
 * CANCELLED status).  With a hook installed (fn != NULL), vocoder_decode,
 * vocoder_decode_windows, vocoder_encode and vocoder_stream_decode call
 * fn(user) on the calling thread before they enqueue any work, and
 * vocoder_decode / vocoder_decode_windows decode their rows in groups of
 * `group` units (decode: rows of the batch, or with tile_frames > 0 time
 * tiles, batch-row major; windows: whole windows with all their sides),
 * wait for each group to finish on the stream and call fn again before the
 * next.  A non-zero return stops the call with VOC_CANCELLED: the groups
 * already decoded are in pcm, the rest of pcm is untouched, and the context
 * (weights, workspace, stream state) stays valid for the next call; a
 * cancelled stream chunk leaves the stream where it was.  Rows are decoded
 * independently, so the samples written equal those of an uncancelled call
 * bit for bit.  Without a hook (fn == NULL, the default) calls stay
 * asynchronous and decode all rows as one batch.
 * Errors: VOC_INVALID_PARAMS (NULL ctx, group < 1).
 */
typedef int (*voc_cancel_fn)(void *user);
voc_status vocoder_set_cancel(voc_ctx *ctx, voc_cancel_fn fn, void *user, int64_t group);

/* Message of the last error on ctx ("" if none); valid until the next call on
 * ctx.  With ctx == NULL, the message of the last failed vocoder_create. */
const char *vocoder_last_error(const voc_ctx *ctx);

/* Release the context, its device weights and workspace.  NULL-safe.  The
 * caller must have synchronized the streams it decoded on. */
void vocoder_destroy(voc_ctx *ctx);

/* ------------------------------------------------------------ profiling
 * When enabled, every kernel launch of the decode, encode and stream calls
 * and of voc_dbg_run_stage
 * is bracketed by two hipEvents recorded on the launch stream, and the
 * algorithmic work of the launch (direct-convolution flops, minimum HBM
 * bytes) is recorded beside them.  vocoder_profile_read synchronizes on the
 * recorded events and returns totals per kernel kind since the last reset. */
typedef enum voc_kernel_kind {
  VOC_K_CONV_IN = 0,  /* conv_in implicit GEMM                          */
  VOC_K_CONVT = 1,    /* polyphase ConvTranspose1d GEMM                 */
  VOC_K_RES_K7 = 2,   /* residual unit conv1 (k=7, dilated) GEMM        */
  VOC_K_RES_K1 = 3,   /* residual unit conv2 (k=1) GEMM + residual add  */
  VOC_K_HEAD = 4,     /* Snake + Conv1d to one or two channels + tanh   */
  VOC_K_IMPORT = 5,   /* latent transpose / tile gather                 */
  VOC_K_EXPORT = 6,   /* debug-stage output transpose                   */
  VOC_K_RES_FUSED = 7, /* whole residual unit (conv1, Snake2, conv2, add) */
  VOC_K_IN_PROJ = 8,  /* dec_in_proj (k=1) GEMM                         */
  VOC_K_ENC_DOWN = 9, /* encoder strided Conv1d GEMM                    */
  VOC_K_ENC_OUT = 10, /* encoder conv_out (k=3) and projection (k=1)    */
  VOC_K_AF_SNAKE = 11, /* alias-free Snake (2x up, Snake, 2x down)      */
  VOC_K_SNAKE = 12,   /* standalone Snake (only in the split ablation)   */
  VOC_K_COL2IM = 13,  /* col2im overlap-add (only in the GEMM + col2im    */
                      /* ablation of the ConvTranspose1d)                 */
  VOC_K_TANH = 14,    /* standalone tanh over the pcm (only in the split  */
                      /* tanh ablation; the head applies tanh otherwise)  */
  VOC_K_COUNT = 15
} voc_kernel_kind;

typedef struct voc_profile_stat {
  int64_t launches;
  double ms;          /* summed event time of the launches               */
  double flops;       /* summed algorithmic flops                        */
  double bytes;       /* summed minimum HBM bytes (inputs+outputs+weights) */
} voc_profile_stat;

voc_status vocoder_profile_enable(voc_ctx *ctx, int enable);
/* Restrict the event pairs to the kinds whose bit (1u << kind) is set in
 * `kinds`; 0 (the default) times every kind.  Launches of other kinds are
 * still counted with their algorithmic work, with ms = 0, and cost no
 * events (events between launches lengthen the gaps between kernels).
 * INVALID_PARAMS for a NULL context or bits at or above VOC_K_COUNT. */
voc_status vocoder_profile_select(voc_ctx *ctx, uint32_t kinds);
voc_status vocoder_profile_reset(voc_ctx *ctx);
voc_status vocoder_profile_read(voc_ctx *ctx, int kind, voc_profile_stat *out);

/* ---------------------------------------------------- debug (not ABI-stable)
 * Stage k of the decoder on caller buffers, for teacher-forced checks:
 *   0 = conv_in (after dec_in_proj when in_proj > 0); for block b: 1 + b*(1+n_res) = Snake + ConvTranspose1d,
 *   the next n_res indices = its residual units; count-1 = the head.
 * in: device fp32 [B, C_in(k), T_in] (stage 0: the latent); out: device fp32
 * [B, C_out(k), T_out] (head: [B, out_channels, T_in]).  Uses the same kernels as
 * vocoder_decode, untiled.  Asynchronous on hip_stream. */
int voc_dbg_stage_count(const voc_ctx *ctx);
voc_status voc_dbg_stage_shape(const voc_ctx *ctx, int stage, int64_t T_in,
                               int64_t *c_in, int64_t *c_out, int64_t *t_out);
voc_status voc_dbg_run_stage(voc_ctx *ctx, int stage, const float *in, int64_t B,
                             int64_t T_in, float *out, void *hip_stream);

/* A plain device-to-device copy of `bytes` bytes (16-byte vector loads and
 * stores), used to calibrate HBM byte counters.  bytes must be a multiple
 * of 16 and both pointers 16-byte aligned. */
voc_status voc_dbg_copy(void *dst, const void *src, int64_t bytes, void *hip_stream);

/* What the device delivers, measured now, beside its published peaks.
 * what = 0: HBM, a plain copy of n bytes (n a multiple of 16; 2 warm-up
 *   copies, then 5 timed): *value = GB/s counting the bytes read and written.
 * what = 1 / 2: matrix cores, n iterations of a loop of 16 independent
 *   16x16 MFMA chains per wave (fp32 16x16x4 / bf16 16x16x32) on 4
 *   workgroups of 4 waves per CU, after a warm-up of n/10: *value = TFLOP/s.
 * what = 3 / 4: the same with 32x32 MFMAs (fp32 32x32x2 / bf16 32x32x16).
 * Allocates its own buffers, runs on hip_stream and synchronizes it; for
 * measurement only, not for a decode loop.  Errors: VOC_INVALID_PARAMS
 * (NULL value, n <= 0, unknown `what`), VOC_DEVICE_ERROR. */
voc_status voc_dbg_peak(int what, int64_t n, double *value, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* VOCODER_H */
