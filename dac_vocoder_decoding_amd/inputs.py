"""Seeded synthetic inputs for the DAC-style decoder: latents and checkpoint tensors.

This module is shared by the HIP path's tests/bench and by the CPU oracle's
tests. It holds no arithmetic of the decoder itself: only the architecture
description (tensor names and shapes), a counter-based random generator and
the value distributions of the synthetic workloads.

Generator (splitmix64 + Box-Muller, per-tensor stream keyed by FNV-1a-64 of
the tensor name).  The pages ("mm3-backend" catalog, trap list) warn that
reproducible noise must come from splitmix64 + Box-Muller rather than a
library normal distribution; the same idea seeds every tensor here:

* stream for tensor ``name`` under ``seed``: ``state0 = seed XOR fnv1a64(name)``;
  the i-th 64-bit draw is ``mix(state0 + (i+1) * 0x9E3779B97F4A7C15)``
  (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014; constants as in Vigna's public splitmix64.c);
* uniform in [0,1): ``(draw >> 11) * 2**-53``;
* normal: one value per pair of uniforms (u1, u2) = (draws 2i, 2i+1):
  ``sqrt(-2 ln(1-u1)) * cos(2 pi u2)`` (Box & Muller 1958);
* values are produced in float64 and rounded to float32; those float32 values
  are "the checkpoint" both implementations consume.

Distributions (the synthetic configurations): latent ~ N(0,1); Snake alpha
(and SnakeBeta beta) ~ U(0.5, 2) per channel; weight-norm magnitude
g ~ U(0.5, 1.5); direction v ~ N(0, 1); every bias ~ N(0, 0.01) read as a
standard deviation of 0.01; the plain dec_in_proj weight (no weight norm)
~ N(0, 1 / C_latent), so its rows have about unit norm like the folded ones.

Tensor naming follows the DAV decoder listing on the minimaxmusic.cpp
ARCHITECTURE page ("Flow VAE" section): dec_in_proj (weight, bias; only
when the configuration has ``in_proj``), conv_in, blocks.{b}.snake1,
blocks.{b}.conv_t1, blocks.{b}.res_units.{r}.{snake1,conv1,snake2,conv2},
snake_out, conv_out, each conv stored as weight_g / weight_v / bias with
PyTorch shapes (Conv1d v: [out, in, k]; ConvTranspose1d v: [in, out, k];
g: [dim0, 1, 1]; Snake alpha: [1, C, 1]).
"""
from __future__ import annotations

import numpy as np

GOLDEN_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1


def fnv1a64(text: str) -> int:
    """FNV-1a 64-bit hash of the UTF-8 bytes of ``text`` (Fowler/Noll/Vo)."""
    h = _FNV_OFFSET
    for byte in text.encode("utf-8"):
        h ^= byte
        h = (h * _FNV_PRIME) & _MASK64
    return h


def splitmix64(state0: int, n: int) -> np.ndarray:
    """The first ``n`` outputs of splitmix64 started from ``state0`` (uint64)."""
    idx = np.arange(1, n + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(state0 & _MASK64) + idx * GOLDEN_GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(state0: int, n: int) -> np.ndarray:
    """n doubles in [0, 1) with 53 random bits each."""
    return (splitmix64(state0, n) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def stream_state(seed: int, name: str) -> int:
    return (seed ^ fnv1a64(name)) & _MASK64


def normal(seed: int, name: str, shape, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    u = uniform01(stream_state(seed, name), 2 * n)
    u1, u2 = u[0::2], u[1::2]
    z = np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * np.pi * u2)
    return (std * z).astype(np.float32).reshape(shape)


def uniform(seed: int, name: str, shape, lo: float, hi: float) -> np.ndarray:
    n = int(np.prod(shape))
    u = uniform01(stream_state(seed, name), n)
    return (lo + (hi - lo) * u).astype(np.float32).reshape(shape)


# --------------------------------------------------------------------------
# Architecture descriptions of the synthetic workloads.
# --------------------------------------------------------------------------

def _cfg(**kw):
    base = dict(latent_channels=64, kernel=7, dilations=(1, 3, 9), act="snake",
                dtype="f32", tile_frames=0, sample_rate=44100, stereo=True)
    base.update(kw)
    base["hop"] = int(np.prod(base["strides"]))
    return base


CONFIGS = {
    0: _cfg(name="tiny_stereo_f32", batch=2, frames=86,
            widths=(256, 128, 64, 32, 16), strides=(8, 8, 4, 2), seed=1000),
    1: _cfg(name="full_stereo_window_f32", batch=2, frames=689,
            widths=(1024, 512, 256, 128, 64), strides=(8, 8, 4, 2), seed=1001),
    2: _cfg(name="batched_windows_bf16", batch=16, frames=689, dtype="bf16",
            widths=(1024, 512, 256, 128, 64), strides=(8, 8, 4, 2), seed=1002),
    3: _cfg(name="long_clip_tiled_snakebeta_f32", batch=2, frames=5168,
            act="snakebeta", tile_frames=512,
            widths=(1024, 512, 256, 128, 64), strides=(8, 8, 4, 2), seed=1003),
    4: _cfg(name="mono_codec_bf16", latent_channels=1024, batch=32, frames=250,
            dtype="bf16", sample_rate=24000, stereo=False,
            widths=(1536, 768, 384, 192, 96), strides=(8, 8, 5, 3), seed=1004),
    # The DAV decoder as the minimaxmusic.cpp ARCHITECTURE page lists it
    # ("Flow VAE"): dec_in_proj 64 -> 1024 (k=1, no weight norm), conv_in
    # 1024 -> 1536, widths 1536 ... 96; one stereo window of 689 frames.
    5: _cfg(name="dav_window_f32", batch=2, frames=689, in_proj=1024,
            widths=(1536, 768, 384, 192, 96), strides=(8, 8, 4, 2), seed=1005),
    # A minute of stereo music through the DAV decoder as the pages' pipeline
    # hands it over ("Inference recipe"): 14 windows of 689 frames (the last
    # 683), each decoded on its own, cropped 86 / 258 frames and stitched.
    6: _cfg(name="dav_song_windows_f32", batch=2, frames=689, in_proj=1024,
            widths=(1536, 768, 384, 192, 96), strides=(8, 8, 4, 2), seed=1006,
            windows=14, last_frames=683, crop=(86, 258)),
    # The causal DAC stage of the Qwen3-TTS codec decoder (qwentts.cpp
    # ARCHITECTURE, "Audio tokenizer decoder": conv_pre 1024 -> 1536, strides
    # 8/5/4/3, widths 1536 ... 96, SnakeBeta, CausalTransConv) streamed as
    # its stateful path does ("Streaming decode"): 32 mono streams of 250
    # frames (5 s at 24 kHz) arriving in chunks of 25 frames.
    7: _cfg(name="causal_codec_stream_bf16", latent_channels=1024, batch=32, frames=250,
            dtype="bf16", sample_rate=24000, stereo=False, act="snakebeta", causal=1,
            widths=(1536, 768, 384, 192, 96), strides=(8, 5, 4, 3), seed=1007, chunk=25),
    # The DAV encoder (minimaxmusic.cpp ARCHITECTURE, "Flow VAE": conv_in
    # 1 -> 64, blocks doubling to 1024 with strides 2/4/8/8, conv_out
    # 1024 -> 1024 k=3, posterior mean 1024 -> 64) on one stereo window:
    # 689 x 512 samples per side -> latent [2, 64, 689].
    8: _cfg(name="dav_encode_window_f32", batch=2, frames=689, in_proj=1024,
            widths=(1536, 768, 384, 192, 96), strides=(8, 8, 4, 2), seed=1008,
            enc_widths=(64, 128, 256, 512, 1024), encode=True),
    # The H3 audio VAE decoder (TensorSharp minimax-h3 page, "audio VAE":
    # DAC/BigVGAN, 32 latent channels -> stereo 32 kHz, upsample rates
    # 5,5,2,2,2,2,2 = 800 samples per 40 Hz latent frame, every nonlinearity
    # alias-free; Snake parameters stored as logs) on the longest clip H3
    # generates, 15 s: latent [1, 32, 600] -> pcm [1, 2, 480000].  Widths
    # halve per block from 2048 to 16 (a reading: the page gives none).
    9: _cfg(name="h3_audio_vae_af_f32", latent_channels=32, batch=1, frames=600,
            sample_rate=32000, act="snakebeta", snake_log_params=1, af_snake=1,
            out_channels=2, widths=(2048, 1024, 512, 256, 128, 64, 32, 16),
            strides=(5, 5, 2, 2, 2, 2, 2), seed=1009),
}


def config(idx: int, **overrides) -> dict:
    """A copy of configuration ``idx`` with fields overridden (e.g. frames, batch)."""
    c = dict(CONFIGS[idx])
    c.update(overrides)
    c["hop"] = int(np.prod(c["strides"]))
    return c


def tensor_shapes(cfg: dict) -> dict:
    """Name -> PyTorch-convention shape of every checkpoint tensor."""
    w = cfg["widths"]
    k = cfg["kernel"]
    cl = cfg["latent_channels"]
    beta = cfg["act"] == "snakebeta"
    shapes = {}

    def conv(prefix, v_shape):
        shapes[prefix + ".weight_v"] = v_shape
        shapes[prefix + ".weight_g"] = (v_shape[0], 1, 1)
        # Conv1d bias has v_shape[0] entries, ConvTranspose1d bias v_shape[1].
        shapes[prefix + ".bias"] = None

    def snake(prefix, c):
        shapes[prefix + ".alpha"] = (1, c, 1)
        if beta:
            shapes[prefix + ".beta"] = (1, c, 1)

    p_in = cfg.get("in_proj", 0)
    if p_in:
        shapes["dec_in_proj.weight"] = (p_in, cl, 1)
        shapes["dec_in_proj.bias"] = (p_in,)
    conv("conv_in", (w[0], p_in or cl, k))
    shapes["conv_in.bias"] = (w[0],)
    for b, s in enumerate(cfg["strides"]):
        cin, cout = w[b], w[b + 1]
        snake(f"blocks.{b}.snake1", cin)
        conv(f"blocks.{b}.conv_t1", (cin, cout, 2 * s))
        shapes[f"blocks.{b}.conv_t1.bias"] = (cout,)
        for r in range(len(cfg["dilations"])):
            p = f"blocks.{b}.res_units.{r}"
            snake(p + ".snake1", cout)
            conv(p + ".conv1", (cout, cout, k))
            shapes[p + ".conv1.bias"] = (cout,)
            snake(p + ".snake2", cout)
            conv(p + ".conv2", (cout, cout, 1))
            shapes[p + ".conv2.bias"] = (cout,)
    snake("snake_out", w[-1])
    nout = cfg.get("out_channels", 1)
    conv("conv_out", (nout, w[-1], k))
    shapes["conv_out.bias"] = (nout,)
    ew = cfg.get("enc_widths")
    if ew:  # the encoder: the decoder's strides in reverse order
        conv("encoder.conv_in", (ew[0], 1, k))
        shapes["encoder.conv_in.bias"] = (ew[0],)
        for b, s in enumerate(reversed(cfg["strides"])):
            q = f"encoder.blocks.{b}"
            for r in range(len(cfg["dilations"])):
                u = f"{q}.res_units.{r}"
                snake(u + ".snake1", ew[b])
                conv(u + ".conv1", (ew[b], ew[b], k))
                shapes[u + ".conv1.bias"] = (ew[b],)
                snake(u + ".snake2", ew[b])
                conv(u + ".conv2", (ew[b], ew[b], 1))
                shapes[u + ".conv2.bias"] = (ew[b],)
            snake(q + ".snake", ew[b])
            conv(q + ".down", (ew[b + 1], ew[b], 2 * s))
            shapes[q + ".down.bias"] = (ew[b + 1],)
        snake("encoder.snake_out", ew[-1])
        conv("encoder.conv_out", (ew[-1], ew[-1], 3))
        shapes["encoder.conv_out.bias"] = (ew[-1],)
        conv("encoder.proj", (cl, ew[-1], 1))
        shapes["encoder.proj.bias"] = (cl,)
    return shapes


def make_weights(cfg: dict, seed: int | None = None, twin: bool = False) -> dict:
    """Seeded float32 checkpoint tensors for ``cfg``.

    ``twin=True`` gives the conditioned twin used for end-to-end gates: the
    same draws, with every residual unit's conv2 magnitude g scaled by 0.3
    (g ~ U(0.15, 0.45)), which keeps the residual stream from growing.
    """
    seed = cfg["seed"] if seed is None else seed
    out = {}
    for name, shape in tensor_shapes(cfg).items():
        if name.endswith(".weight_v"):
            out[name] = normal(seed, name, shape)
        elif name == "dec_in_proj.weight":
            out[name] = normal(seed, name, shape, std=float(1.0 / np.sqrt(shape[1])))
        elif name.endswith(".weight_g"):
            if twin and ".res_units." in name and ".conv2." in name:
                n = int(np.prod(shape))
                u = uniform01(stream_state(seed, name), n)
                out[name] = (0.3 * (0.5 + u)).astype(np.float32).reshape(shape)
            else:
                out[name] = uniform(seed, name, shape, 0.5, 1.5)
        elif name.endswith(".bias"):
            out[name] = normal(seed, name, shape, std=0.01)
        elif name.endswith(".alpha") or name.endswith(".beta"):
            out[name] = uniform(seed, name, shape, 0.5, 2.0)
            if cfg.get("snake_log_params", 0):  # stored as logs of the same draws
                out[name] = np.log(out[name].astype(np.float64)).astype(np.float32)
        else:  # pragma: no cover
            raise KeyError(name)
    return out


def make_windows(cfg: dict, seed: int | None = None, windows: int | None = None,
                 frames: int | None = None, last_frames: int | None = None) -> np.ndarray:
    """Seeded latent windows [n, sides * C_latent, L] ~ N(0, 1), float32, one
    independent draw per window (the pages' denoiser produces each window on
    its own); the last window's frames from ``last_frames`` on are zero.
    sides is 2 for a stereo pair of latents, 1 for a mono latent or one that
    decodes to both channels."""
    seed = cfg["seed"] if seed is None else seed
    n = cfg["windows"] if windows is None else windows
    L = cfg["frames"] if frames is None else frames
    last = cfg["last_frames"] if last_frames is None else last_frames
    sides = 2 if cfg["stereo"] and cfg.get("out_channels", 1) == 1 else 1
    x = normal(seed, "windows", (n, sides * cfg["latent_channels"], L))
    x[-1, :, last:] = 0.0
    return x


def make_latent(cfg: dict, seed: int | None = None, batch: int | None = None,
                frames: int | None = None) -> np.ndarray:
    """Seeded latent [B, C_latent, T] ~ N(0, 1), float32."""
    seed = cfg["seed"] if seed is None else seed
    b = cfg["batch"] if batch is None else batch
    t = cfg["frames"] if frames is None else frames
    return normal(seed, "latent", (b, cfg["latent_channels"], t))


def make_audio(cfg: dict, seed: int | None = None, batch: int | None = None,
               frames: int | None = None) -> np.ndarray:
    """Seeded audio [B, 1, frames * hop] ~ 0.5 * N(0, 1), float32 (music-like
    level: unit-variance noise scaled to an RMS of 0.5)."""
    seed = cfg["seed"] if seed is None else seed
    b = cfg["batch"] if batch is None else batch
    t = cfg["frames"] if frames is None else frames
    return normal(seed, "audio", (b, 1, t * cfg["hop"]), std=0.5)


def audio_seconds(cfg: dict, batch: int, frames: int) -> float:
    """Decoded audio-seconds: stereo pairs count once (two rows per stereo
    second, or one row when the decoder writes both channels)."""
    samples = frames * cfg["hop"]
    rows = batch / 2 if cfg["stereo"] and cfg.get("out_channels", 1) == 1 else batch
    return rows * samples / cfg["sample_rate"]


def encode_flops(cfg: dict, batch: int, frames: int) -> float:
    """Direct-convolution multiply-adds x 2 of one encode of frames * hop samples."""
    ew, k = cfg["enc_widths"], cfg["kernel"]
    t = frames * cfg["hop"]
    f = 2.0 * batch * t * ew[0] * k
    for b, s in enumerate(reversed(cfg["strides"])):
        for _ in cfg["dilations"]:
            f += 2.0 * batch * t * ew[b] * ew[b] * (k + 1)
        t //= s
        f += 2.0 * batch * t * ew[b + 1] * ew[b] * 2 * s
    f += 2.0 * batch * t * ew[-1] * ew[-1] * 3 + 2.0 * batch * t * cfg["latent_channels"] * ew[-1]
    return f


def algorithmic_flops(cfg: dict, batch: int, frames: int) -> float:
    """Direct-convolution multiply-adds x 2 for one decode (no im2col, no zero-stuffing)."""
    w = cfg["widths"]
    k = cfg["kernel"]
    t = frames
    cin = cfg["latent_channels"]
    f = 0.0
    if cfg.get("in_proj", 0):
        f += 2.0 * batch * t * cfg["in_proj"] * cin
        cin = cfg["in_proj"]
    f += 2.0 * batch * t * w[0] * cin * k
    for b, s in enumerate(cfg["strides"]):
        cin, cout = w[b], w[b + 1]
        f += 2.0 * batch * t * cin * cout * 2 * s  # every input frame meets 2s taps
        t *= s
        for _ in cfg["dilations"]:
            f += 2.0 * batch * t * cout * cout * k + 2.0 * batch * t * cout * cout
    f += 2.0 * batch * t * w[-1] * k * cfg.get("out_channels", 1)
    return f


def af_elements(cfg: dict, batch: int, frames: int) -> float:
    """Activation elements that pass through a Snake in one decode (each one
    alias-free Snake output element in an af_snake configuration)."""
    w, t, n = cfg["widths"], frames, 0.0
    for b, s in enumerate(cfg["strides"]):
        n += batch * t * w[b]                            # the block's Snake
        t *= s
        n += batch * t * w[b + 1] * 2 * len(cfg["dilations"])
    return n + batch * t * w[-1]                         # snake_out
