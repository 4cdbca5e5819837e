"""GPU parity of the alias-free decoder (the H3 audio VAE of the TensorSharp
minimax-h3 page: every Snake inside a 2x upsample / Snake / 2x downsample
sandwich, Snake parameters stored as logs, 32 latent channels to two output
channels, rates 5,5,2,2,2,2,2):

* every stage against the oracle on the GPU's own input (fp32; bf16 against
  the oracle that rounds the same operands, and the exact one);
* whole decodes against the oracle (conditioned twin weights);
* the alias-free Snake kernel's edges: rows of 1 to 40 frames (runs of 16
  frames per thread, replicate padding at both ends) and rows of different
  lengths in one launch (ragged windows);
* time tiles with the exact 30-frame halo equal the untiled decode bit for
  bit, and windowed decodes write both output channels planar.
"""
import numpy as np
import pytest
import torch

from dac_vocoder_decoding_amd import inputs as I
from dac_vocoder_decoding_amd import vocoder as V
from oracle import oracle as O

from gpu_util import BF16_E2E_MAXABS_WIDE, TOL, bf16_stage_ok, rel_maxabs, rel_rms, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    V.lib()


def small(dtype="f32", **kw):
    """The H3 decoder's rates and channel counts at small widths."""
    widths = (64, 32, 32, 32, 32, 32, 16, 16) if dtype == "f32" else (64,) + (32,) * 7
    return I.config(9, dtype=dtype, widths=widths, **kw)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_af_stages_vs_oracle(dtype):
    cfg = small(dtype)
    t = I.make_weights(cfg)
    lat = I.make_latent(cfg, batch=2, frames=3)
    ctx = V.open_context(cfg, t)
    try:
        m = O.Model(cfg, t)
        mr = O.Model(cfg, t, round_operands=True)
        x = to_dev(lat)
        for k in range(V.voc_dbg_stage_count(ctx)):
            y = V.run_stage(ctx, k, x)
            torch.cuda.synchronize()
            xin, got = x.cpu().numpy(), y.cpu().numpy()
            ref = m.run_stage(k, xin)
            e = rel_maxabs(got, ref)
            if dtype == "f32":
                assert e <= TOL["f32"], (k, e)
            else:
                ref_r = mr.run_stage(k, xin)
                floor = rel_maxabs(ref_r, ref)
                print(f"stage {k}: GPU {e:.2e}, bf16 operand floor {floor:.2e}")
                assert bf16_stage_ok(e, floor), (k, e, floor)
                assert rel_rms(got, ref_r) <= 1e-3, (k, rel_rms(got, ref_r))
            x = y
    finally:
        V.vocoder_destroy(ctx)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_af_decode_vs_oracle(dtype):
    cfg = small(dtype)
    t = I.make_weights(cfg, twin=True)
    lat = I.make_latent(cfg, batch=2, frames=7)
    ctx = V.open_context(cfg, t)
    try:
        pcm = V.decode(ctx, to_dev(lat)).cpu().numpy()
    finally:
        V.vocoder_destroy(ctx)
    ref = O.Model(cfg, t).decode(lat)
    assert pcm.shape == ref.shape == (2, 2, 7 * 800)
    e_max, e_rms = rel_maxabs(pcm, ref), rel_rms(pcm, ref)
    # The page reports its own port's audio VAE decode at cosine similarity
    # 0.999995 to its reference; the fp32 decode here must do at least as well.
    cos = float(np.sum(pcm * ref) / np.sqrt(np.sum(pcm ** 2) * np.sum(ref ** 2)))
    print(f"alias-free {dtype}: max-abs/RMS {e_max:.2e} rel-RMS {e_rms:.2e} cosine {cos:.9f}")
    if dtype == "f32":
        assert e_max <= TOL["f32"]
        assert cos >= 0.999995
    else:
        assert e_rms <= TOL["bf16"]
        assert e_max <= BF16_E2E_MAXABS_WIDE, e_max


@pytest.mark.parametrize("T", [1, 2, 3, 5, 15, 16, 17, 33, 40])
def test_af_kernel_row_lengths(T):
    """The block-0 stage (alias-free Snake, then ConvTranspose1d) and the last
    residual unit of block 0 on rows of T frames: every run split, short rows
    where both replicate pads meet, exact against the oracle."""
    cfg = small()
    t = I.make_weights(cfg)
    ctx = V.open_context(cfg, t)
    try:
        m = O.Model(cfg, t)
        for k in (1, 4):
            c_in = V.voc_dbg_stage_shape(ctx, k, T)[1]
            x = I.normal(T, f"stage{k}", (3, c_in, T))
            y = V.run_stage(ctx, k, to_dev(x)).cpu().numpy()
            e = rel_maxabs(y, m.run_stage(k, x))
            assert e <= TOL["f32"], (k, T, e)
    finally:
        V.vocoder_destroy(ctx)


def test_af_windows_two_channels_ragged():
    """Windows of different lengths in one launch (the last one ragged), each
    window's rows replicate-padded at its own ends; both output channels
    written planar."""
    cfg = small()
    t = I.make_weights(cfg, twin=True)
    win = I.make_windows(cfg, windows=3, frames=9, last_frames=4)
    ctx = V.open_context(cfg, t)
    try:
        pcm = V.decode_windows(ctx, to_dev(win), 1, 4, 2, 3).cpu().numpy()
    finally:
        V.vocoder_destroy(ctx)
    ref = O.Model(cfg, t).decode_windows(win, 4, 2, 3)
    assert pcm.shape == ref.shape == (2, (6 + 4 + 2) * 800)
    assert rel_maxabs(pcm, ref) <= TOL["f32"]


def test_af_tiles_equal_untiled():
    cfg = small()
    t = I.make_weights(cfg, twin=True)
    lat = I.make_latent(cfg, batch=2, frames=75)
    assert V.voc_config_halo(V.config_from_dict(cfg)) == 30
    x = to_dev(lat)
    outs = []
    for tile in (0, 16, 29):
        ctx = V.open_context(cfg, t, tile_frames=tile)
        try:
            outs.append(V.decode(ctx, x))
            torch.cuda.synchronize()
        finally:
            V.vocoder_destroy(ctx)
    assert torch.equal(outs[1], outs[0]) and torch.equal(outs[2], outs[0])


def test_af_log_params_match_plain_params():
    """snake_log_params=1 with log-stored parameters decodes like the plain
    parameters (exp at load, in double precision)."""
    cfg = small()
    t = I.make_weights(cfg, twin=True)                       # logs (the H3 convention)
    plain = dict(t)
    for k in t:
        if k.endswith(".alpha") or k.endswith(".beta"):
            plain[k] = np.exp(t[k].astype(np.float64)).astype(np.float32)
    lat = to_dev(I.make_latent(cfg, batch=1, frames=5))
    a = V.open_context(cfg, t)
    b = V.open_context(cfg, plain, snake_log_params=0)
    try:
        ya, yb = V.decode(a, lat), V.decode(b, lat)
        torch.cuda.synchronize()
    finally:
        V.vocoder_destroy(a)
        V.vocoder_destroy(b)
    assert float((ya - yb).abs().max()) <= 1e-5


@pytest.mark.parametrize("T", [1, 2, 5])
def test_af_decode_short_clips(T):
    """Clips of 1, 2 and 5 latent frames: every alias-free Snake's replicate
    padding meets both row ends within one run."""
    cfg = small()
    t = I.make_weights(cfg, twin=True)
    lat = I.make_latent(cfg, batch=1, frames=T)
    ctx = V.open_context(cfg, t)
    try:
        pcm = V.decode(ctx, to_dev(lat)).cpu().numpy()
    finally:
        V.vocoder_destroy(ctx)
    ref = O.Model(cfg, t).decode(lat)
    assert pcm.shape == ref.shape == (1, 2, T * 800)
    assert rel_maxabs(pcm, ref) <= TOL["f32"]
