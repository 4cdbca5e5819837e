"""vocoder_decode_noalloc: the decode for callers that cannot allocate,
with its workspace in the library's fixed per-GPU scratch array, checked
bit for bit against vocoder_decode on two calls in a row (the second with
a smaller input), across contexts that share the array, with the workspace
allocator capped so that any allocation would fail, and rejecting a
configuration that cannot fit one latent frame."""
import pytest
import torch

from dac_vocoder_decoding_amd import inputs as I
from dac_vocoder_decoding_amd import vocoder as V

from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def _noalloc(ctx, x):
    b, c, t = x.shape
    V.expect_dim("latent", x.shape, 1, V.latent_channels(ctx))
    pcm = torch.full((b, V.out_channels(ctx), V.vocoder_output_length(ctx, t)), 7.0, device=x.device)
    V.check(V.vocoder_decode_noalloc(ctx, x, b, t, pcm), ctx)
    return pcm


@pytest.mark.parametrize("idx,shapes,terms", [
    (1, [(2, 689), (2, 100)], 1),     # full window: tiled into passes; then one pass
    (0, [(2, 86), (1, 9)], 1),
    (2, [(16, 689), (4, 40)], 1),     # bf16 batched windows
    (2, [(16, 689), (4, 40)], 2),     # the same with two-term operands (twice the operand planes)
    (3, [(2, 1200), (2, 300)], 1),    # SnakeBeta with 512-frame tiles
])
def test_noalloc_equals_decode_on_two_calls(idx, shapes, terms, monkeypatch):
    cfg = I.config(idx)
    t = I.make_weights(cfg, twin=True)
    lats = [to_dev(I.make_latent(cfg, batch=b, frames=n)) for b, n in shapes]
    kw = {"operand_terms": 2} if terms == 2 else {}
    ctx = V.open_context(cfg, t, **kw)
    try:
        refs = [V.decode(ctx, x) for x in lats]
        torch.cuda.synchronize()
    finally:
        V.vocoder_destroy(ctx)
    # A context whose workspace allocator is capped at one byte: any
    # allocation on the decode path would fail with VOC_OOM.
    monkeypatch.setenv("VOC_MAX_WORKSPACE_BYTES", "1")
    ctx = V.open_context(cfg, t, **kw)
    try:
        for x, ref in zip(lats, refs):
            got = _noalloc(ctx, x)
            torch.cuda.synchronize()
            assert torch.equal(got, ref)
        with pytest.raises(V.VocError) as ei:     # the allocating path is refused
            V.decode(ctx, lats[-1])
        assert ei.value.status == V.VOC_OOM
    finally:
        V.vocoder_destroy(ctx)


def test_noalloc_contexts_share_the_scratch():
    a_cfg, b_cfg = I.config(0), I.config(5)
    ta, tb = I.make_weights(a_cfg, twin=True), I.make_weights(b_cfg, twin=True)
    xa = to_dev(I.make_latent(a_cfg, batch=2, frames=40))
    xb = to_dev(I.make_latent(b_cfg, batch=2, frames=30))
    a, b = V.open_context(a_cfg, ta), V.open_context(b_cfg, tb)
    try:
        ra, rb = V.decode(a, xa), V.decode(b, xb)
        ga1 = _noalloc(a, xa)
        gb = _noalloc(b, xb)
        ga2 = _noalloc(a, xa)
        torch.cuda.synchronize()
        assert torch.equal(ga1, ra) and torch.equal(gb, rb) and torch.equal(ga2, ra)
    finally:
        V.vocoder_destroy(a)
        V.vocoder_destroy(b)


def test_noalloc_rejects_a_frame_beyond_the_scratch():
    # 16 channels at a hop of 2^20 samples: one latent frame's activations
    # alone take 16 x 2^20 x 4 bytes per buffer, more than 256 MiB together.
    cfg = I.config(0, widths=(16, 16, 16, 16, 16), strides=(64, 64, 64, 4), latent_channels=16)
    ctx = V.open_context(cfg, I.make_weights(cfg, twin=True))
    try:
        x = torch.zeros(1, 16, 1, device="cuda")
        pcm = torch.zeros(1, 1, cfg["hop"], device="cuda")
        assert V.vocoder_decode_noalloc(ctx, x, 1, 1, pcm) == V.VOC_INVALID_PARAMS
        assert "no-allocation scratch" in V.vocoder_last_error(ctx)
    finally:
        V.vocoder_destroy(ctx)
