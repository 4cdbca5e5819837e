"""GPU parity of the windowed decode with stitching (vocoder_decode_windows)
on the DAV decoder (dec_in_proj 64 -> 1024, conv_in 1024 -> 1536, widths
1536 ... 96):

* small windows against the oracle's windowed decode (fp32 and bf16);
* windows cut from one continuous track, with crops wider than the
  receptive-field halo, against the GPU's own decode of the whole track, at
  small size and at the full size of the minute-long song (14 windows of
  689 frames, crops 86 / 258);
* argument checks and output lengths, rejected on the host before any kernel.
"""
import numpy as np
import pytest
import torch

from dac_vocoder_decoding_amd import inputs as I
from dac_vocoder_decoding_amd import vocoder as V
from oracle import oracle as O

from gpu_util import BF16_E2E_MAXABS, TOL, rel_maxabs, rel_rms, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    V.lib()


def _cut_windows(track, L, step):
    """Windows of L frames every `step` frames of one track [sides*C, T], the
    last one ending at the track's end: (windows [n, sides*C, L], its length)."""
    T = track.shape[1]
    starts = [0]
    while starts[-1] + L < T:
        starts.append(starts[-1] + step)
    out = np.zeros((len(starts), track.shape[0], L), dtype=np.float32)
    for k, s0 in enumerate(starts):
        seg = track[:, s0:s0 + L]
        out[k, :, :seg.shape[1]] = seg
    return out, T - starts[-1]


@pytest.mark.parametrize("idx", [5, 2])
def test_windows_parity_vs_oracle(idx):
    """Three small stereo windows (the last one ragged) through the GPU and the
    oracle; fp32 max-abs within 1e-4 of the RMS, bf16 relative RMS within 2e-2."""
    cfg = I.config(idx)
    t = I.make_weights(cfg, twin=True)
    win = I.make_windows(cfg, windows=3, frames=12, last_frames=10)
    ctx = V.open_context(cfg, t)
    try:
        pcm = V.decode_windows(ctx, to_dev(win), 2, 10, 3, 4).cpu().numpy()
        assert V.vocoder_windows_output_length(ctx, 3, 12, 10, 3, 4) == (8 + 5 + 7) * cfg["hop"]
    finally:
        V.vocoder_destroy(ctx)
    ref = O.Model(cfg, t).decode_windows(win, 10, 3, 4)
    assert pcm.shape == ref.shape == (2, 20 * cfg["hop"])
    e_max, e_rms = rel_maxabs(pcm, ref), rel_rms(pcm, ref)
    print(f"cfg{idx} windows: max-abs/RMS {e_max:.2e} rel-RMS {e_rms:.2e}")
    if cfg["dtype"] == "f32":
        assert e_max <= TOL["f32"]
    else:
        assert e_rms <= TOL["bf16"]
        assert e_max <= BF16_E2E_MAXABS, e_max


def test_windows_mono():
    cfg = I.config(5, stereo=False)
    t = I.make_weights(cfg, twin=True)
    win = I.make_windows(cfg, windows=2, frames=9, last_frames=9)
    ctx = V.open_context(cfg, t)
    try:
        pcm = V.decode_windows(ctx, to_dev(win), 1, 9, 2, 3).cpu().numpy()
    finally:
        V.vocoder_destroy(ctx)
    ref = O.Model(cfg, t).decode_windows(win, 9, 2, 3)
    assert pcm.shape == ref.shape == (1, (6 + 7) * cfg["hop"])
    assert rel_maxabs(pcm, ref) <= TOL["f32"]


def _track_case(cfg, t, T, L, cl, cr):
    track = I.normal(cfg["seed"], "track", (2 * cfg["latent_channels"], T))
    win, last = _cut_windows(track, L, L - cl - cr)
    ctx = V.open_context(cfg, t)
    try:
        stitched = V.decode_windows(ctx, to_dev(win), 2, last, cl, cr)
        whole = V.decode(ctx, to_dev(track.reshape(2, cfg["latent_channels"], T)))[:, 0, :]
        torch.cuda.synchronize()
    finally:
        V.vocoder_destroy(ctx)
    return stitched, whole, win.shape[0]


def test_windows_cut_from_one_track_equal_its_decode():
    cfg = I.config(5)
    t = I.make_weights(cfg, twin=True)
    stitched, whole, n = _track_case(cfg, t, 100, 40, 12, 14)
    assert n == 6 and stitched.shape == whole.shape
    err = float((stitched - whole).abs().max())
    print(f"windows vs whole-track decode: max abs {err:.2e}")
    assert torch.equal(stitched, whole)


def test_fullsize_song_windows_equal_the_track_decode():
    """The minute-long song at full size: 14 windows of 689 frames cut 345
    frames apart from one 5168-frame track stitch back to the track's decode."""
    cfg = I.config(6)
    t = I.make_weights(cfg)
    L, (cl, cr) = cfg["frames"], cfg["crop"]
    stitched, whole, n = _track_case(cfg, t, 5168, L, cl, cr)
    assert n == cfg["windows"] == 14
    assert stitched.shape == (2, 5168 * cfg["hop"])
    assert bool(torch.isfinite(stitched).all()) and float(stitched.abs().max()) <= 1.0
    err = float((stitched - whole).abs().max())
    print(f"song windows vs whole-track decode: max abs {err:.2e}")
    assert torch.equal(stitched, whole)


def test_windows_argument_checks():
    cfg = I.config(5)
    t = I.make_weights(cfg)
    ctx = V.open_context(cfg, t)
    x = torch.zeros(3, 128, 12, device="cuda")
    y = torch.zeros(2, 64 * 512, device="cuda")
    try:
        L = V.vocoder_windows_output_length
        assert L(ctx, 14, 689, 683, 86, 258) == 5168 * 512      # the song: no gap, no overlap
        assert L(ctx, 1, 689, 689, 86, 258) == 689 * 512        # one window keeps all
        assert L(ctx, 2, 689, 87, 86, 258) == (431 + 1) * 512
        for bad in [(0, 12, 12, 3, 4), (3, 12, 13, 3, 4), (3, 12, 0, 3, 4), (3, 12, 12, -1, 4),
                    (3, 12, 12, 6, 6), (2, 12, 3, 3, 4), (2, 12, 12, 0, 12)]:
            assert L(ctx, *bad) == -1, bad
            n, Lw, last, cl, cr = bad
            assert V.vocoder_decode_windows(ctx, x, n, 2, Lw, last, cl, cr, y) == V.VOC_INVALID_PARAMS
        assert V.vocoder_decode_windows(ctx, x, 3, 3, 12, 12, 3, 4, y) == V.VOC_INVALID_PARAMS
        assert V.vocoder_decode_windows(ctx, None, 3, 2, 12, 12, 3, 4, y) == V.VOC_INVALID_PARAMS
        assert V.vocoder_decode_windows(ctx, x, 3, 0, 12, 12, 3, 4, y) == V.VOC_INVALID_PARAMS
        assert "sides" in V.vocoder_last_error(ctx)
    finally:
        V.vocoder_destroy(ctx)
    tiled = V.open_context(cfg, t, tile_frames=16)
    try:
        assert V.vocoder_decode_windows(tiled, x, 3, 2, 12, 12, 3, 4, y) == V.VOC_INVALID_PARAMS
        assert "tile_frames" in V.vocoder_last_error(tiled)
    finally:
        V.vocoder_destroy(tiled)


def test_stereo_windows_with_two_output_channels():
    """sides = 2 and two output channels per side: planes (side, channel) in
    the order j * 2 + o, against the oracle's windowed decode."""
    cfg = I.config(5, out_channels=2, widths=(256, 128, 64, 32, 16), in_proj=0)
    t = I.make_weights(cfg, twin=True)
    win = I.normal(cfg["seed"], "win2", (3, 2 * cfg["latent_channels"], 10))
    win[-1, :, 7:] = 0.0
    ctx = V.open_context(cfg, t)
    try:
        pcm = V.decode_windows(ctx, to_dev(win), 2, 7, 2, 3).cpu().numpy()
    finally:
        V.vocoder_destroy(ctx)
    ref = O.Model(cfg, t).decode_windows(win, 7, 2, 3)
    assert pcm.shape == ref.shape == (4, (7 + 5 + 5) * cfg["hop"])
    assert rel_maxabs(pcm, ref) <= TOL["f32"]
