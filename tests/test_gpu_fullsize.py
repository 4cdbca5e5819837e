"""Parity at the full sizes of the synthetic single-decode workloads (the
windowed song is covered in test_gpu_windows.py), in the launch
configuration the benchmark times.  The oracle cannot decode these whole in
seconds, so it computes sampled outputs exactly:

* per stage (teacher forcing): the GPU's own stage input, cut to a window
  with the stage's receptive-field margin, through the oracle stage; the
  window's interior is exact, start and ragged end windows include the true
  clip edges;
* end to end (conditioned twin): the oracle decodes latent windows with the
  exact halo (10 frames; 20 on the left for the causal stack; 30 for the
  alias-free H3 decoder), which reproduces the untiled decode on the
  window's own samples (pinned in the oracle tests);
plus properties that hold at any size (length, tanh range, L != R, tiled =
untiled bitwise for the long clip)."""
import numpy as np
import pytest
import torch

from dac_vocoder_decoding_amd import inputs as I
from dac_vocoder_decoding_amd import vocoder as V
from oracle import oracle as O

from gpu_util import TOL, oracle_stage_window, rel_maxabs, rel_rms, to_dev, windows

pytestmark = pytest.mark.gpu

@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4, 5, 7, 9])
def test_fullsize_stage_parity_sampled(idx):
    cfg = I.config(idx)
    t = I.make_weights(cfg)
    lat = I.make_latent(cfg)
    B = cfg["batch"]
    rows = sorted({0, B - 1})
    ctx = V.open_context(cfg, t, tile_frames=0)
    try:
        m = O.Model(cfg, t)
        x = to_dev(lat)
        worst = 0.0
        for k in range(V.voc_dbg_stage_count(ctx)):
            y = V.run_stage(ctx, k, x)
            torch.cuda.synchronize()
            t_in = x.shape[-1]
            w = 24 if k == 0 else 12
            for a, e in windows(t_in, w):
                ref, sl = oracle_stage_window(m, k, x, rows, a, e)
                got = y[rows, :, sl].cpu().numpy()
                err = rel_maxabs(got, ref)
                worst = max(worst, err)
                assert err <= TOL[cfg["dtype"]], (k, a, e, err)
            x = y
        print(f"cfg{idx}: worst sampled stage error {worst:.2e}")
    finally:
        V.vocoder_destroy(ctx)


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4, 5, 7, 9])
def test_fullsize_twin_decode_sampled(idx):
    cfg = I.config(idx)
    t = I.make_weights(cfg, twin=True)
    lat = I.make_latent(cfg)
    B, T, hop = cfg["batch"], cfg["frames"], cfg["hop"]
    ctx = V.open_context(cfg, t)
    try:
        pcm = V.decode(ctx, to_dev(lat))
        torch.cuda.synchronize()
    finally:
        V.vocoder_destroy(ctx)
    m = O.Model(cfg, t)
    w = 2 if idx in (4, 7) else 3
    cases = [(0, 0, w), (B - 1, T - w, T)]
    if cfg["tile_frames"]:   # a tile seam: frames around 512
        cases.append((1, cfg["tile_frames"] - 2, cfg["tile_frames"] + 1))
    halo_l = V.voc_config_halo(V.config_from_dict(cfg))   # the left halo when causal
    halo_r = 0 if cfg.get("causal") else halo_l
    for r, t0, t1 in cases:
        a, e = max(0, t0 - halo_l), min(T, t1 + halo_r)
        ref = m.decode(lat[r:r + 1, :, a:e])[0, :, (t0 - a) * hop:(t1 - a) * hop]
        got = pcm[r, :, t0 * hop:t1 * hop].cpu().numpy()
        e_max, e_rms = rel_maxabs(got, ref), rel_rms(got, ref)
        print(f"cfg{idx} twin row {r} frames [{t0},{t1}): max-abs/RMS {e_max:.2e} rel-RMS {e_rms:.2e}")
        if cfg["dtype"] == "f32":
            assert e_max <= TOL["f32"]
        else:
            assert e_rms <= TOL["bf16"]


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4, 5, 7, 9])
def test_fullsize_literal_invariants(idx):
    cfg = I.config(idx)
    t = I.make_weights(cfg)
    lat = I.make_latent(cfg)
    ctx = V.open_context(cfg, t)
    try:
        pcm = V.decode(ctx, to_dev(lat))
        torch.cuda.synchronize()
    finally:
        V.vocoder_destroy(ctx)
    B, T, O = cfg["batch"], cfg["frames"], cfg.get("out_channels", 1)
    assert pcm.shape == (B, O, T * cfg["hop"])
    assert bool(torch.isfinite(pcm).all()) and float(pcm.abs().max()) <= 1.0
    assert float(pcm.pow(2).mean().sqrt()) > 1e-2
    if O == 2:                                   # one row decodes to stereo
        lr = (pcm[:, 0] - pcm[:, 1]).abs().amax(dim=-1)
        assert float(lr.min()) > 1e-3
    elif cfg["stereo"]:
        lr = (pcm[0::2] - pcm[1::2]).abs().amax(dim=-1)
        assert float(lr.min()) > 1e-3            # left differs from right


def test_fullsize_long_clip_tiled_equals_untiled():
    cfg = I.config(3)
    t = I.make_weights(cfg)
    lat = I.make_latent(cfg)
    x = to_dev(lat)
    a = V.open_context(cfg, t)                    # tiles of 512 frames
    try:
        ya = V.decode(a, x)
        torch.cuda.synchronize()
    finally:
        V.vocoder_destroy(a)
    b = V.open_context(cfg, t, tile_frames=0)
    try:
        yb = V.decode(b, x)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb)
    finally:
        V.vocoder_destroy(b)
