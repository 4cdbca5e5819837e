"""CPU oracle of the DAC-style waveform decoder -- TEST INFRASTRUCTURE ONLY.

Only tests/, ``__graft_entry__.smoke()`` and bench.py's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding)
never imports or calls it, and this module imports nothing from the product.

The arithmetic lives in ``oracle.c`` (direct loops; fp64 build = the oracle,
fp32 build = the precision floor).  This file only orders the steps of the
decoder the way the pages state them and holds the readings of points the
pages leave open.

Decoder (minimaxmusic.cpp ARCHITECTURE, "Flow VAE" listing; DAV decoder):
    x = dec_in_proj(latent)        (DAV only)            Conv1d k1, bias, no weight norm
    h = conv_in(x)                                       Conv1d k7, pad 3, bias
    for each block b (stride s):
        h = conv_t1(Snake_b(h))                          ConvTranspose1d k=2s, stride s
        for d in (1, 3, 9):                              residual units
            h = h + conv2(Snake2(conv1_d(Snake1(h))))    conv1 k7 dilation d, conv2 k1
    pcm = tanh(conv_out(Snake_out(h)))                   Conv1d k7 -> 1 channel, bias

Readings of points the pages leave open (each listed in the design notes):
  * conv padding is zero "same" padding (K-1)/2*d, so the residual add lines up;
  * ConvTranspose1d keeps full[n + ceil(s/2)] for n in [0, T*s): for even s
    this is the pages' "pad s/2"; for odd s it is PyTorch padding=ceil(s/2),
    output_padding=1;
  * the convT weight norm is taken along axis 0 of the stored [in, out, k]
    tensor (per input channel), as the pages' "axis 0" says literally;
  * Snake denominators are alpha + 1e-9 (Snake) and beta + 1e-9 (SnakeBeta);
  * every conv has a bias, dec_in_proj included; N(0, 0.01) biases use std
    0.01;
  * dec_in_proj feeds conv_in directly (the listing puts no activation
    between them), and its output is zero-padded like any conv input;
  * causal configurations (qwentts.cpp ARCHITECTURE, "Audio tokenizer
    decoder": CausalTransConv, and "Streaming decode (stateful path)": every
    module causal, state cleared to zero at reset = the offline zero left
    pads): every k=7 conv (conv_in, residual conv1, conv_out) pads (K-1)*d on
    the left only, and the transposed conv keeps full[n] for n in [0, T*s)
    (its K - s = s tail on the right is what a stream carries into the next
    frame);
  * windowed decode (ARCHITECTURE, "Inference recipe": "Decode and stitch",
    "Post-processing"): windows are decoded independently, every window but
    the first loses crop_left latent frames (x hop samples) on the left, every
    window but the last crop_right on the right, the kept segments are
    concatenated in window order and clamped to [-1, 1]; stereo output is
    planar [L: N][R: N];
  * bf16 configurations: the folded weights are rounded fp64 -> fp32 (the F32
    inference checkpoint) -> bf16 (round to nearest even), the latent is
    rounded to bf16, and everything else stays exact.  Optionally
    (``round_operands=True``) the input of every matrix-core convolution
    (conv_in, ConvTranspose1d, residual conv1 and conv2) after its Snake is
    also rounded to bf16, mirroring an implementation whose matrix-core
    operands are bf16 while accumulation and the residual stream stay wide;
    the output head (a contraction to one channel) keeps its input wide.
    With ``operand_terms=2`` those operands are rounded to two bf16 terms
    instead (hi = bf16(x), lo = bf16(x - hi), carried as hi + lo): the
    reading of an implementation that multiplies both terms by the same
    weights;

Pins (tests/test_oracle_pins.py) hold every function here to closed forms,
brute force, textbook/library routines and invariants the pages fix.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
# VOC_ORACLE_LIBDIR names a directory holding other builds of oracle.c under
# the same file names (the sanitizer test builds them with ASan and UBSan);
# those are loaded as they are, never rebuilt.
_LIBDIR = os.environ.get("VOC_ORACLE_LIBDIR")
_LIBS = {"f64": os.path.join(_LIBDIR or _HERE, "liboracle_f64.so"),
         "f32": os.path.join(_LIBDIR or _HERE, "liboracle_f32.so")}
_DEFS = {"f64": ["-DREAL=double"], "f32": ["-DREAL=float", "-DORACLE_FLOAT"]}
_NP = {"f64": np.float64, "f32": np.float32}
_loaded = {}


def build_library() -> None:
    """Compile both builds of oracle.c with gcc (OpenMP, no fast-math)."""
    for prec, out in _LIBS.items():
        compile_library(_SRC, out + ".tmp", prec)
        os.replace(out + ".tmp", out)


def load_library(path: str, prec: str):
    """Load one build of oracle.c and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P, I = ctypes.c_void_p, ctypes.c_int64
    lib.orc_real_size.restype = ctypes.c_int
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_snake.argtypes = [P, P, I, I, I, P, P]
    lib.orc_weight_norm.argtypes = [P, P, P, I, I, P]
    lib.orc_conv1d.argtypes = [P, P, I, I, I, P, P, I, I, I, I]
    lib.orc_conv_transpose1d.argtypes = [P, P, I, I, I, P, P, I, I, I, I, I]
    lib.orc_conv1d_strided.argtypes = [P, P, I, I, I, P, P, I, I, I, I, I]
    lib.orc_tanh.argtypes = [P, P, I]
    lib.orc_add.argtypes = [P, P, P, I]
    assert lib.orc_real_size() == np.dtype(_NP[prec]).itemsize
    return lib


def compile_library(src: str, out: str, prec: str = "f64", extra=()) -> None:
    """Compile a C source with the oracle's flags (used for both builds);
    `extra` adds flags (e.g. the sanitizers)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-fno-fast-math", "-ffp-contract=off", *_DEFS[prec], *extra, src, "-o", out, "-lm"]
    subprocess.check_call(cmd)


def _lib(prec: str):
    if prec not in _loaded:
        path = _LIBS[prec]
        if not _LIBDIR and (not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC)):
            build_library()
        _loaded[prec] = load_library(path, prec)
    return _loaded[prec]


def _c(a, prec):
    return np.ascontiguousarray(a, dtype=_NP[prec])


def _p(a):
    return None if a is None else a.ctypes.data


# --------------------------------------------------------------------------
# Primitive operations (each a direct loop in oracle.c).
# --------------------------------------------------------------------------

def snake(x, alpha, beta=None, prec="f64"):
    """Snake(x) = x + sin^2(alpha x)/(alpha+1e-9); SnakeBeta uses beta+1e-9. x: [R, C, T]."""
    x = _c(x, prec)
    r, c, t = x.shape
    a = _c(np.reshape(alpha, -1), prec)
    b = None if beta is None else _c(np.reshape(beta, -1), prec)
    assert a.size == c and (b is None or b.size == c)
    y = np.empty_like(x)
    _lib(prec).orc_snake(_p(x), _p(y), r, c, t, _p(a), _p(b))
    return y


def weight_norm(v, g, prec="f64"):
    """Fold w = g * v / ||v|| along axis 0 of v.  Returns (w, norms)."""
    v = _c(v, prec)
    g = _c(np.reshape(g, -1), prec)
    d0 = v.shape[0]
    assert g.size == d0
    w = np.empty_like(v)
    n = np.empty(d0, dtype=_NP[prec])
    _lib(prec).orc_weight_norm(_p(v), _p(g), _p(w), d0, v.size // d0, _p(n))
    return w, n


def conv1d(x, w, bias=None, dilation=1, prec="f64", causal=False):
    """Zero-padded Conv1d keeping the length.  x: [R, Cin, T], w: [Cout, Cin, K]
    (K odd).  'same' padding (K-1)/2*d each side, or causal: (K-1)*d on the left."""
    x = _c(x, prec)
    w = _c(w, prec)
    r, cin, t = x.shape
    cout, cin2, k = w.shape
    assert cin == cin2 and k % 2 == 1
    pad = (k - 1) * dilation if causal else (k - 1) // 2 * dilation
    b = None if bias is None else _c(np.reshape(bias, -1), prec)
    y = np.empty((r, cout, t), dtype=_NP[prec])
    _lib(prec).orc_conv1d(_p(x), _p(y), r, cin, t, _p(w), _p(b), cout, k, dilation, pad)
    return y


def conv1d_strided(x, w, bias, stride, pad, prec="f64"):
    """Strided Conv1d with zero padding `pad` on both sides.  x: [R, Cin, T],
    w: [Cout, Cin, K]; output length (T + 2 pad - K) // stride + 1."""
    x = _c(x, prec)
    w = _c(w, prec)
    r, cin, t = x.shape
    cout, cin2, k = w.shape
    assert cin == cin2
    tout = (t + 2 * pad - k) // stride + 1
    b = None if bias is None else _c(np.reshape(bias, -1), prec)
    y = np.empty((r, cout, tout), dtype=_NP[prec])
    _lib(prec).orc_conv1d_strided(_p(x), _p(y), r, cin, t, _p(w), _p(b), cout, k, stride, pad, tout)
    return y


def convt_crop(stride: int, causal: bool = False) -> int:
    """Left crop of the transposed conv: ceil(s/2) (s/2 for even s), or 0 for
    the causal transposed conv (which drops the K - s tail on the right)."""
    return 0 if causal else (stride + 1) // 2


def conv_transpose1d(x, w, bias, stride, pad_left=None, out_len=None, prec="f64"):
    """ConvTranspose1d.  x: [R, Cin, T], w: [Cin, Cout, K]; keeps full[n+pad_left], n < out_len."""
    x = _c(x, prec)
    w = _c(w, prec)
    r, cin, t = x.shape
    cin2, cout, k = w.shape
    assert cin == cin2
    p = convt_crop(stride) if pad_left is None else pad_left
    tout = t * stride if out_len is None else out_len
    b = None if bias is None else _c(np.reshape(bias, -1), prec)
    y = np.empty((r, cout, tout), dtype=_NP[prec])
    _lib(prec).orc_conv_transpose1d(_p(x), _p(y), r, cin, t, _p(w), _p(b), cout, k,
                                    stride, p, tout)
    return y


def tanh(x, prec="f64"):
    x = _c(x, prec)
    y = np.empty_like(x)
    _lib(prec).orc_tanh(_p(x), _p(y), x.size)
    return y


def add(a, b, prec="f64"):
    a = _c(a, prec)
    b = _c(b, prec)
    assert a.shape == b.shape
    y = np.empty_like(a)
    _lib(prec).orc_add(_p(a), _p(b), _p(y), a.size)
    return y


# --------------------------------------------------------------------------
# Alias-free Snake (TensorSharp minimax-h3.md: the H3 audio VAE wraps every
# nonlinearity in a 2x upsample / activate / 2x downsample sandwich).  The
# page gives no filter; the reading is the textbook windowed-sinc low-pass:
# a Kaiser window (Kaiser's beta for the attenuation of the transition
# band), 12 taps, cutoff at half the original Nyquist, transition half-width
# 0.3 of it, normalised to unit DC gain, replicate padding at the clip ends.
# --------------------------------------------------------------------------
AF_TAPS = 12


def kaiser_beta(atten_db: float) -> float:
    """Kaiser's window parameter for a stop-band attenuation of atten_db."""
    if atten_db > 50.0:
        return 0.1102 * (atten_db - 8.7)
    if atten_db >= 21.0:
        return 0.5842 * (atten_db - 21.0) ** 0.4 + 0.07886 * (atten_db - 21.0)
    return 0.0


def af_filter(taps: int = AF_TAPS, cutoff: float = 0.25, half_width: float = 0.3) -> np.ndarray:
    """Kaiser-windowed sinc low-pass, even length, centred between taps
    (cutoff and half_width in cycles per sample at the 2x rate)."""
    half = taps // 2
    atten = 2.285 * (half - 1) * np.pi * (4.0 * half_width) + 7.95
    beta = kaiser_beta(atten)
    n = np.arange(taps)
    window = np.i0(beta * np.sqrt(1.0 - ((2.0 * n) / (taps - 1) - 1.0) ** 2)) / np.i0(beta)
    t = np.arange(-half, half) + 0.5
    f = 2.0 * cutoff * window * np.sinc(2.0 * cutoff * t)
    return f / f.sum()


def upsample2(x, f=None):
    """x [R, C, T] -> [R, C, 2T]: replicate-pad by half the taps / 2, insert a
    zero after every sample, filter with 2 f (unit DC gain at the 2x rate),
    keep the 2T samples aligned with x."""
    f = af_filter() if f is None else f
    k = f.size
    pad = k // 2 - 1                              # 5 input samples each side
    x = np.asarray(x, dtype=np.float64)
    r, c, t = x.shape
    xp = np.concatenate([np.repeat(x[:, :, :1], pad, 2), x, np.repeat(x[:, :, -1:], pad, 2)], axis=2)
    z = np.zeros((r, c, 2 * xp.shape[2]))
    z[:, :, ::2] = xp
    full = np.zeros((r, c, z.shape[2] + k - 1))
    for j in range(k):                            # full[n] = sum_j 2 f[j] z[n - j]
        full[:, :, j:j + z.shape[2]] += 2.0 * f[j] * z
    lo = 2 * pad + (k - 2) // 2                   # 15: the sample aligned with x[0]
    return full[:, :, lo:lo + 2 * t]


def downsample2(v, f=None):
    """v [R, C, 2T] -> [R, C, T]: replicate-pad k/2 - 1 left and k/2 right,
    filter with f and keep every second sample."""
    f = af_filter() if f is None else f
    k = f.size
    v = np.asarray(v, dtype=np.float64)
    n2 = v.shape[2]
    vp = np.concatenate([np.repeat(v[:, :, :1], k // 2 - 1, 2), v, np.repeat(v[:, :, -1:], k // 2, 2)], axis=2)
    out = np.zeros(v.shape[:2] + (n2 // 2,))
    for j in range(k):                            # out[t] = sum_j f[j] vp[2t + j]
        out += f[j] * vp[:, :, j:j + n2:2]
    return out


def af_snake(x, alpha, beta=None, prec="f64"):
    """down2(Snake(up2(x))), per channel."""
    u = upsample2(x)
    return _c(downsample2(snake(u, alpha, beta, "f64")), prec)


def round_bf16(x) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even) via float32; returns float64.

    bf16 keeps the top 16 bits of an IEEE float32: add 0x7FFF plus the lowest
    kept bit, then truncate.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def round_bf16_two_term(x) -> np.ndarray:
    """x as two bf16 terms: hi = bf16(x) and lo = bf16(x - hi), returned as
    hi + lo in float64 (the value a two-term matrix-core operand carries:
    both terms meet the same weights).  x is taken at float32, as the
    operands are formed in float32."""
    x32 = np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)
    hi = round_bf16(x32)
    lo = round_bf16((x32 - hi).astype(np.float32))
    return hi + lo


# --------------------------------------------------------------------------
# The decoder.
# --------------------------------------------------------------------------

class Model:
    """Folded weights of one decoder, held at the oracle's precision."""

    def __init__(self, cfg: dict, tensors: dict, prec: str = "f64",
                 bf16: bool | None = None, round_operands: bool = False, operand_terms: int = 1):
        self.cfg = cfg
        self.prec = prec
        self.bf16 = (cfg["dtype"] == "bf16") if bf16 is None else bf16
        self.round_operands = round_operands and self.bf16
        # round_operands with two terms: each operand is rounded to the pair
        # hi + lo of bf16 values instead of one bf16 value.
        self._round_op = round_bf16_two_term if operand_terms == 2 else round_bf16
        self.beta = cfg["act"] == "snakebeta"
        self.causal = bool(cfg.get("causal", 0))
        self.af = bool(cfg.get("af_snake", 0))
        self.norms = {}
        t = tensors

        def fold(prefix):
            # The fold is always fp64 (it is done once at conversion).
            w, n = weight_norm(t[prefix + ".weight_v"], t[prefix + ".weight_g"], "f64")
            self.norms[prefix] = n
            if self.bf16:
                w = round_bf16(w.astype(np.float32))
            return _c(w, prec)

        def vec(name):
            return _c(np.reshape(t[name], -1), prec)

        # Snake parameters stored as logs (the H3 audio VAE of the TensorSharp
        # minimax-h3 page keeps alpha and beta in log scale) are exponentiated
        # once, at load.
        log_params = bool(cfg.get("snake_log_params", 0))

        def act(prefix):
            def p(name):
                v = np.reshape(np.asarray(t[name], dtype=np.float64), -1)
                return _c(np.exp(v) if log_params else v, prec)
            return (p(prefix + ".alpha"), p(prefix + ".beta") if self.beta else None)

        # dec_in_proj is stored without weight norm: used as given (bf16
        # configurations round it fp32 -> bf16 like the folded weights).
        self.in_proj = None
        if cfg.get("in_proj", 0):
            w = np.asarray(t["dec_in_proj.weight"], dtype=np.float32)
            w = round_bf16(w) if self.bf16 else w
            self.in_proj = (_c(w, prec), vec("dec_in_proj.bias"))
        self.conv_in = (fold("conv_in"), vec("conv_in.bias"))
        self.blocks = []
        for b, s in enumerate(cfg["strides"]):
            p = f"blocks.{b}"
            units = []
            for r, d in enumerate(cfg["dilations"]):
                q = f"{p}.res_units.{r}"
                units.append(dict(d=d, act1=act(q + ".snake1"),
                                  w1=fold(q + ".conv1"), b1=vec(q + ".conv1.bias"),
                                  act2=act(q + ".snake2"),
                                  w2=fold(q + ".conv2"), b2=vec(q + ".conv2.bias")))
            self.blocks.append(dict(s=s, act=act(p + ".snake1"),
                                    wt=fold(p + ".conv_t1"), bt=vec(p + ".conv_t1.bias"),
                                    units=units))
        self.head = (act("snake_out"), fold("conv_out"), vec("conv_out.bias"))

    # ---- stages -----------------------------------------------------------
    def _snake(self, x, a, operand=True):
        """Snake (alias-free when configured); in round_operands mode a
        matrix-core operand is rounded to bf16."""
        y = af_snake(x, a[0], a[1], self.prec) if self.af else snake(x, a[0], a[1], self.prec)
        if self.round_operands and operand:
            y = _c(self._round_op(y), self.prec)
        return y

    def _latent(self, latent):
        x = np.asarray(latent, dtype=np.float32)
        return _c(round_bf16(x) if self.bf16 else x, self.prec)

    def stage_conv_in(self, latent):
        x = self._latent(latent)
        if self.in_proj is not None:
            x = conv1d(x, self.in_proj[0], self.in_proj[1], 1, self.prec)
            if self.round_operands:  # conv_in's matrix-core operand
                x = _c(self._round_op(x), self.prec)
        w, b = self.conv_in
        return conv1d(x, w, b, 1, self.prec, self.causal)

    def stage_upsample(self, b, h):
        blk = self.blocks[b]
        return conv_transpose1d(self._snake(h, blk["act"]), blk["wt"], blk["bt"], blk["s"],
                                pad_left=convt_crop(blk["s"], self.causal), prec=self.prec)

    def stage_res_unit(self, b, r, h):
        u = self.blocks[b]["units"][r]
        v = conv1d(self._snake(h, u["act1"]), u["w1"], u["b1"], u["d"], self.prec, self.causal)
        return add(h, conv1d(self._snake(v, u["act2"]), u["w2"], u["b2"], 1, self.prec),
                   self.prec)

    def stage_head_pre(self, h):
        # The head contracts to one output channel: no matrix-core operand,
        # so its Snake output is not rounded even in round_operands mode.
        a, w, b = self.head
        return conv1d(self._snake(h, a, operand=False), w, b, 1, self.prec, self.causal)

    def stage_head(self, h):
        return tanh(self.stage_head_pre(h), self.prec)

    # Stage numbering shared with the debug stage runner of the library:
    # 0 = conv_in; then per block b: 1 + b*(1+n_res) = Snake + ConvTranspose1d,
    # the next n_res indices = residual units; last = head.
    def n_stages(self):
        return 2 + len(self.blocks) * (1 + len(self.cfg["dilations"]))

    def run_stage(self, k, x):
        nr = len(self.cfg["dilations"])
        if k == 0:
            return self.stage_conv_in(x)
        if k == self.n_stages() - 1:
            return self.stage_head(x)
        b, j = divmod(k - 1, 1 + nr)
        return self.stage_upsample(b, x) if j == 0 else self.stage_res_unit(b, j - 1, x)

    def decode(self, latent, pre_tanh=False):
        """latent [B, C_latent, T] -> pcm [B, out_channels, T*hop] (or the pre-tanh value)."""
        h = self.stage_conv_in(latent)
        for b in range(len(self.blocks)):
            h = self.stage_upsample(b, h)
            for r in range(len(self.cfg["dilations"])):
                h = self.stage_res_unit(b, r, h)
        return self.stage_head_pre(h) if pre_tanh else self.stage_head(h)

    def decode_windows(self, windows, last_frames, crop_left, crop_right):
        """Windowed decode and stitch.  windows [n, sides*C, L]: side j of
        window k is channels [j*C, (j+1)*C); the last window holds
        last_frames frames.  Returns planar [sides * out_channels, N] (output
        channel o of side j in plane j * out_channels + o), clamped to [-1, 1]."""
        windows = np.asarray(windows)
        n, sc, L = windows.shape
        c = self.cfg["latent_channels"]
        sides = sc // c
        hop = self.cfg["hop"]
        segments = []
        for k in range(n):
            length = last_frames if k == n - 1 else L
            x = windows[k, :, :length].reshape(sides, c, length)
            y = self.decode(x)                               # [sides, O, length*hop]
            y = y.reshape(-1, y.shape[-1])                   # plane j*O + o
            lo = crop_left if k > 0 else 0
            hi = length - (crop_right if k < n - 1 else 0)
            assert hi > lo, "every window must keep at least one frame"
            segments.append(y[:, lo * hop:hi * hop])
        return np.clip(np.concatenate(segments, axis=1), -1.0, 1.0)

    def decode_tiled(self, latent, tile, halo):
        """Decode latent frames [t0, t1) of each tile from the window
        [t0 - halo, t1 + halo) clamped to the clip, keeping the tile's own
        samples.  Equals decode() when halo covers the receptive field."""
        latent = np.asarray(latent)
        bsz, _, t = latent.shape
        hop = self.cfg["hop"]
        out = np.empty((bsz, self.head[1].shape[0], t * hop), dtype=_NP[self.prec])
        for t0 in range(0, t, tile):
            t1 = min(t, t0 + tile)
            a, e = max(0, t0 - halo), min(t, t1 + halo)
            y = self.decode(latent[:, :, a:e])
            out[:, :, t0 * hop:t1 * hop] = y[:, :, (t0 - a) * hop:(t1 - a) * hop]
        return out


class Encoder:
    """The DAV encoder (minimaxmusic.cpp ARCHITECTURE, "Flow VAE": the mirror
    of the decoder), per side:
        h = conv_in(audio)                          Conv1d 1 -> E0, k=7, "same" padding
        for each block b (stride s = the decoder's strides reversed):
            h = residual units (dilations 1, 3, 9) at width E_b
            h = down(Snake(h))                      Conv1d E_b -> E_{b+1}, k=2s, stride s, pad s/2
        z = conv_out(Snake_out(h))                  Conv1d k=3, "same" padding
        mean = proj(z)                              Conv1d k=1 to the latent channels
    Readings: every encoder conv is weight-normed (the page says all convs
    of the checkpoint are); no activation between conv_out and proj; the
    encode is the posterior mean (the page: deterministic, no sampling)."""

    def __init__(self, cfg: dict, tensors: dict, prec: str = "f64", round_operands: bool = False):
        self.cfg = cfg
        self.prec = prec
        self.bf16 = cfg["dtype"] == "bf16"
        self.round_operands = round_operands and self.bf16
        self.beta = cfg["act"] == "snakebeta"
        t = tensors

        def fold(prefix):
            w, _ = weight_norm(t[prefix + ".weight_v"], t[prefix + ".weight_g"], "f64")
            if self.bf16:
                w = round_bf16(w.astype(np.float32))
            return _c(w, prec)

        def vec(name):
            return _c(np.reshape(t[name], -1), prec)

        def act(prefix):
            return (vec(prefix + ".alpha"), vec(prefix + ".beta") if self.beta else None)

        p = "encoder"
        self.conv_in = (fold(p + ".conv_in"), vec(p + ".conv_in.bias"))
        self.blocks = []
        for b, s in enumerate(reversed(cfg["strides"])):
            q = f"{p}.blocks.{b}"
            units = []
            for r, d in enumerate(cfg["dilations"]):
                u = f"{q}.res_units.{r}"
                units.append(dict(d=d, act1=act(u + ".snake1"), w1=fold(u + ".conv1"),
                                  b1=vec(u + ".conv1.bias"), act2=act(u + ".snake2"),
                                  w2=fold(u + ".conv2"), b2=vec(u + ".conv2.bias")))
            self.blocks.append(dict(s=s, units=units, act=act(q + ".snake"),
                                    wd=fold(q + ".down"), bd=vec(q + ".down.bias")))
        self.out = (act(p + ".snake_out"), fold(p + ".conv_out"), vec(p + ".conv_out.bias"))
        self.proj = (fold(p + ".proj"), vec(p + ".proj.bias"))

    def _op(self, y):
        return _c(round_bf16(y), self.prec) if self.round_operands else y

    def _snake(self, x, a):
        return self._op(snake(x, a[0], a[1], self.prec))

    def encode(self, audio):
        """audio [B, 1, T*hop] -> posterior mean [B, C_latent, T]."""
        x = np.asarray(audio, dtype=np.float32)
        x = _c(round_bf16(x) if self.bf16 else x, self.prec)
        h = conv1d(x, self.conv_in[0], self.conv_in[1], 1, self.prec)
        for blk in self.blocks:
            for u in blk["units"]:
                v = conv1d(self._snake(h, u["act1"]), u["w1"], u["b1"], u["d"], self.prec)
                h = add(h, conv1d(self._snake(v, u["act2"]), u["w2"], u["b2"], 1, self.prec), self.prec)
            s = blk["s"]
            h = conv1d_strided(self._snake(h, blk["act"]), blk["wd"], blk["bd"], s, s // 2, self.prec)
        a, w, b = self.out
        z = conv1d(self._snake(h, a), w, b, 1, self.prec)
        return conv1d(self._op(z), self.proj[0], self.proj[1], 1, self.prec)


def num_threads(prec: str = "f64") -> int:
    """Threads the oracle's OpenMP loops use."""
    return _lib(prec).orc_num_threads()
