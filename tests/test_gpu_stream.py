"""GPU checks of the causal decoder and its streaming decode (the causal DAC
stage of the Qwen3-TTS codec decoder: conv_pre 1024 -> 1536, strides
8/5/4/3, widths 1536 ... 96, SnakeBeta):

* causal stages and whole decodes against the oracle, fp32 and bf16;
* a stream fed chunk by chunk (chunks of 1 to 25 frames) reproduces the
  offline decode of the concatenated latent bit for bit, at small size and
  at the full size of 32 streams of 250 frames;
* causal time tiles (left halo only) equal the untiled decode bit for bit;
* argument checks, rejected on the host before any kernel.
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


def _stream(ctx, lat, chunks):
    """Feed lat [rows, C, T] through the stream in the given chunk sizes."""
    rows, _, T = lat.shape
    assert sum(chunks) == T
    V.check(V.vocoder_stream_reset(ctx, rows), ctx)
    out, t0 = [], 0
    for t in chunks:
        out.append(V.stream_decode(ctx, lat[:, :, t0:t0 + t].contiguous()))
        t0 += t
    torch.cuda.synchronize()
    return torch.cat(out, dim=-1)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_causal_stages_and_decode_vs_oracle(dtype):
    cfg = I.config(7, dtype=dtype)
    t = I.make_weights(cfg, twin=True)
    lat = I.make_latent(cfg, batch=2, frames=6)
    ctx = V.open_context(cfg, t)
    try:
        m = O.Model(cfg, t)
        x = to_dev(lat)
        for k in range(V.voc_dbg_stage_count(ctx)):
            y = V.run_stage(ctx, k, x)
            torch.cuda.synchronize()
            e = rel_maxabs(y.cpu().numpy(), m.run_stage(k, x.cpu().numpy()))
            assert e <= TOL[dtype], (k, e)
            x = y
        pcm = V.decode(ctx, to_dev(lat)).cpu().numpy()
    finally:
        V.vocoder_destroy(ctx)
    ref = m.decode(lat)
    e_max, e_rms = rel_maxabs(pcm, ref), rel_rms(pcm, ref)
    print(f"causal {dtype}: max-abs/RMS {e_max:.2e} rel-RMS {e_rms:.2e}")
    if dtype == "f32":
        assert e_max <= TOL["f32"]
    else:
        assert e_rms <= TOL["bf16"]
        assert e_max <= BF16_E2E_MAXABS_WIDE, e_max


def test_causal_literal_bf16_stages_vs_floor():
    """Literal weights, bf16, every stage on the GPU's own input.  Against the
    oracle that rounds the same operands to bf16 the kernels must agree
    closely (rel-RMS <= 1e-3, max-abs <= 1e-2 of the stage RMS).  Against the
    exact oracle the bf16 operands alone cost up to 2.05e-2 of the RMS on
    this workload (the operand-rounded oracle's own error), so the 2e-2 gate
    is held where that floor leaves room and the floor plus 1e-3 elsewhere
    (bf16_stage_ok)."""
    cfg = I.config(7)
    t = I.make_weights(cfg)
    lat = I.make_latent(cfg, batch=2, frames=4)
    ctx = V.open_context(cfg, t)
    try:
        m = O.Model(cfg, t)
        mr = O.Model(cfg, t, round_operands=True)
        x = to_dev(lat)
        for k in range(V.voc_dbg_stage_count(ctx)):
            y = V.run_stage(ctx, k, x)
            torch.cuda.synchronize()
            xin, got = x.cpu().numpy(), y.cpu().numpy()
            ref, ref_r = m.run_stage(k, xin), mr.run_stage(k, xin)
            floor = rel_maxabs(ref_r, ref)
            e = rel_maxabs(got, ref)
            print(f"stage {k}: GPU {e:.2e}, bf16 operand floor {floor:.2e}")
            assert bf16_stage_ok(e, floor), (k, e, floor)
            assert rel_rms(got, ref_r) <= 1e-3, (k, rel_rms(got, ref_r))
            assert rel_maxabs(got, ref_r) <= 1e-2, (k, rel_maxabs(got, ref_r))
            x = y
    finally:
        V.vocoder_destroy(ctx)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stream_equals_offline_bitwise(dtype):
    cfg = I.config(7, dtype=dtype)
    t = I.make_weights(cfg, twin=True)
    lat = I.make_latent(cfg, batch=3, frames=60)
    ctx = V.open_context(cfg, t)
    try:
        x = to_dev(lat)
        offline = V.decode(ctx, x)
        for chunks in ([1] * 30 + [30], [25, 25, 10], [7, 1, 13, 2, 20, 17], [60]):
            got = _stream(ctx, x, chunks)
            assert got.shape == offline.shape
            assert torch.equal(got, offline), chunks
        # A reset starts over: the same stream again gives the same samples.
        assert torch.equal(_stream(ctx, x, [25, 25, 10]), offline)
    finally:
        V.vocoder_destroy(ctx)
    if dtype == "f32":
        ref = O.Model(cfg, t).decode(lat)
        assert rel_maxabs(offline.cpu().numpy(), ref) <= TOL["f32"]


def test_fullsize_stream_equals_offline():
    """32 streams of 250 frames in chunks of 25 (the streaming workload)."""
    cfg = I.config(7)
    t = I.make_weights(cfg)
    lat = I.make_latent(cfg)
    ctx = V.open_context(cfg, t)
    try:
        x = to_dev(lat)
        offline = V.decode(ctx, x)
        got = _stream(ctx, x, [cfg["chunk"]] * (cfg["frames"] // cfg["chunk"]))
    finally:
        V.vocoder_destroy(ctx)
    assert got.shape == (32, 1, 250 * 480)
    assert bool(torch.isfinite(got).all()) and float(got.abs().max()) <= 1.0
    assert torch.equal(got, offline)


def test_causal_tiles_equal_untiled():
    cfg = I.config(7, dtype="f32")
    t = I.make_weights(cfg, twin=True)
    lat = I.make_latent(cfg, batch=2, frames=70)
    x = to_dev(lat)
    outs = []
    for tile in (0, 16, 23):
        ctx = V.open_context(cfg, t, tile_frames=tile)
        try:
            outs.append(V.decode(ctx, x))
            torch.cuda.synchronize()
        finally:
            V.vocoder_destroy(ctx)
    assert torch.equal(outs[1], outs[0]) and torch.equal(outs[2], outs[0])


def test_stream_argument_checks():
    cfg = I.config(7, dtype="f32")
    t = I.make_weights(cfg)
    x = torch.zeros(2, 1024, 4, device="cuda")
    y = torch.zeros(2, 1, 4 * 480, device="cuda")
    ctx = V.open_context(cfg, t)
    try:
        assert V.vocoder_stream_decode(ctx, x, 4, y) == V.VOC_INVALID_PARAMS   # no reset yet
        assert "reset" in V.vocoder_last_error(ctx)
        assert V.vocoder_stream_reset(ctx, 0) == V.VOC_INVALID_PARAMS
        assert V.vocoder_stream_reset(ctx, 2) == V.VOC_OK
        assert V.vocoder_stream_decode(ctx, x, 0, y) == V.VOC_INVALID_PARAMS
        assert V.vocoder_stream_decode(ctx, None, 4, y) == V.VOC_INVALID_PARAMS
        assert V.vocoder_stream_decode(ctx, x, 4, y) == V.VOC_OK
        torch.cuda.synchronize()
    finally:
        V.vocoder_destroy(ctx)
    centered = V.open_context(I.config(4), I.make_weights(I.config(4)))
    try:
        assert V.vocoder_stream_reset(centered, 2) == V.VOC_INVALID_PARAMS
        assert "causal" in V.vocoder_last_error(centered)
    finally:
        V.vocoder_destroy(centered)


def test_two_channel_causal_stream():
    """A causal decoder with two output channels: the stream writes both
    channels of every chunk, equal bit for bit to the offline decode, which
    matches the oracle."""
    cfg = I.config(7, dtype="f32", widths=(64, 32, 32, 32, 32), latent_channels=32, out_channels=2)
    t = I.make_weights(cfg, twin=True)
    lat = I.make_latent(cfg, batch=2, frames=30)
    ctx = V.open_context(cfg, t)
    try:
        x = to_dev(lat)
        offline = V.decode(ctx, x)
        got = _stream(ctx, x, [7, 1, 12, 10])
    finally:
        V.vocoder_destroy(ctx)
    assert offline.shape == (2, 2, 30 * cfg["hop"])
    assert torch.equal(got, offline)
    ref = O.Model(cfg, t).decode(lat)
    assert rel_maxabs(offline.cpu().numpy(), ref) <= TOL["f32"]
