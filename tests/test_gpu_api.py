"""The C ABI's behaviour on a device: weight validation (all-or-nothing),
decode argument checks, the workspace cap, and the per-launch profiler's
accounting.  Every failing call here is rejected on the host before any
kernel runs."""
import os

import numpy as np
import pytest
import torch

from dac_vocoder_decoding_amd import inputs as I
from dac_vocoder_decoding_amd import vocoder as V

from gpu_util import to_dev

pytestmark = pytest.mark.gpu

CFG = I.config(0)


@pytest.fixture(scope="module")
def weights():
    return I.make_weights(CFG, twin=True)


def _create(**kw):
    st, ctx = V.vocoder_create(V.config_from_dict({**CFG, **kw}), 0)
    assert st == V.VOC_OK, V.vocoder_last_error(None)
    return ctx


def test_decode_before_load_is_rejected():
    ctx = _create()
    try:
        x = torch.zeros(2, 64, 4, device="cuda")
        y = torch.zeros(2, 1, 4 * 512, device="cuda")
        assert V.vocoder_decode(ctx, x, 2, 4, y) == V.VOC_NOT_LOADED
        assert "not loaded" in V.vocoder_last_error(ctx)
    finally:
        V.vocoder_destroy(ctx)


@pytest.mark.parametrize("mutate,needle", [
    (lambda t: t.pop("conv_in.bias"), "missing"),
    (lambda t: t.__setitem__("blocks.9.snake1.alpha", np.ones(4, np.float32)), "unknown"),
    (lambda t: t.__setitem__("conv_in.weight_v", np.ones((256, 64, 5), np.float32)), "shape"),
    (lambda t: t["blocks.1.conv_t1.bias"].__setitem__(3, np.nan), "non-finite"),
    (lambda t: t["blocks.2.res_units.1.conv1.weight_v"].__setitem__((5, slice(None), slice(None)), 0.0),
     "||v||"),
    (lambda t: t["blocks.0.res_units.0.conv2.weight_v"].__setitem__((1, 2, 0), np.inf), "||v||"),
])
def test_bad_weights_rejected_and_previous_weights_kept(weights, mutate, needle):
    ctx = _create()
    try:
        assert V.vocoder_load_weights(ctx, weights) == V.VOC_OK
        x = to_dev(I.make_latent(CFG, batch=2, frames=5))
        before = V.decode(ctx, x)
        bad = {k: v.copy() for k, v in weights.items()}
        mutate(bad)
        assert V.vocoder_load_weights(ctx, bad) == V.VOC_BAD_WEIGHTS
        assert needle in V.vocoder_last_error(ctx)
        after = V.decode(ctx, x)
        torch.cuda.synchronize()
        assert torch.equal(before, after)
    finally:
        V.vocoder_destroy(ctx)


def test_squeezed_shapes_accepted(weights):
    ctx = _create()
    try:
        sq = {k: (v.reshape(-1) if v.ndim == 3 and v.shape[1] == 1 else v) for k, v in weights.items()}
        sq = {k: (v.reshape(v.shape[1]) if k.endswith(".alpha") else v) for k, v in sq.items()}
        assert V.vocoder_load_weights(ctx, sq) == V.VOC_OK
    finally:
        V.vocoder_destroy(ctx)


def test_decode_argument_checks(weights):
    ctx = V.open_context(CFG, weights)
    try:
        x = torch.zeros(2, 64, 4, device="cuda")
        y = torch.zeros(2, 1, 4 * 512 + 4, device="cuda")
        assert V.vocoder_decode(ctx, x, 0, 4, y) == V.VOC_INVALID_PARAMS
        assert V.vocoder_decode(ctx, x, 2, 0, y) == V.VOC_INVALID_PARAMS
        assert V.vocoder_decode(ctx, None, 2, 4, y) == V.VOC_INVALID_PARAMS
        assert V.vocoder_decode(ctx, x.data_ptr() + 4, 2, 4, y) == V.VOC_INVALID_PARAMS
        assert V.vocoder_decode(ctx, x, 2, 4, y.data_ptr() + 8) == V.VOC_INVALID_PARAMS
        # Size limits, rejected before any allocation or kernel: a row of
        # 2^31 samples, and more than 65535 rows.
        assert V.vocoder_decode(ctx, x, 2, 1 << 22, y) == V.VOC_INVALID_PARAMS
        assert "2^31" in V.vocoder_last_error(ctx)
        assert V.vocoder_decode(ctx, x, 70000, 4, y) == V.VOC_INVALID_PARAMS
        assert "rows" in V.vocoder_last_error(ctx)
        assert V.vocoder_output_length(ctx, 7) == 7 * 512
        assert V.voc_dbg_run_stage(ctx, 99, x, 2, 4, y) == V.VOC_INVALID_PARAMS
    finally:
        V.vocoder_destroy(ctx)


def test_workspace_cap_gives_oom(weights, monkeypatch):
    monkeypatch.setenv("VOC_MAX_WORKSPACE_BYTES", str(1 << 20))
    ctx = V.open_context(CFG, weights)
    monkeypatch.delenv("VOC_MAX_WORKSPACE_BYTES")
    try:
        x = to_dev(I.make_latent(CFG, batch=2, frames=40))
        y = torch.empty(2, 1, 40 * 512, device="cuda")
        assert V.vocoder_decode(ctx, x, 2, 40, y) == V.VOC_OOM
        assert "VOC_MAX_WORKSPACE_BYTES" in V.vocoder_last_error(ctx)
    finally:
        V.vocoder_destroy(ctx)


def test_profiler_accounting(weights):
    ctx = V.open_context(CFG, weights)
    try:
        B, T = 2, 30
        x = to_dev(I.make_latent(CFG, batch=B, frames=T))
        V.decode(ctx, x)
        V.check(V.vocoder_profile_reset(ctx))
        V.check(V.vocoder_profile_enable(ctx, True))
        for _ in range(3):
            V.decode(ctx, x)
        V.check(V.vocoder_profile_enable(ctx, False))
        stats = {}
        for k, n in enumerate(V.KERNEL_KINDS):
            st, s = V.vocoder_profile_read(ctx, k)
            assert st == V.VOC_OK
            stats[n] = s
        expect = {"conv_in": 1, "convt": 4, "head": 1, "import": 1}
        for n, c in expect.items():
            assert stats[n]["launches"] == 3 * c, n
            assert stats[n]["ms"] > 0
        # Each residual unit runs either fused or as a conv1 + conv2 pair.
        fused = stats["res_fused"]["launches"]
        assert stats["res_k7"]["launches"] + fused == 3 * 12
        assert stats["res_k1"]["launches"] + fused == 3 * 12
        total = sum(stats[n]["flops"] for n in
                    ("conv_in", "convt", "res_k7", "res_k1", "head", "res_fused"))
        assert abs(total / 3 - I.algorithmic_flops(CFG, B, T)) <= 1e-9 * total
    finally:
        V.vocoder_destroy(ctx)


def test_copy_kernel_and_stream_argument():
    src = torch.arange(4096, dtype=torch.float32, device="cuda")
    dst = torch.zeros_like(src)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        assert V.voc_dbg_copy(dst, src, 4096 * 4, s) == V.VOC_OK
    s.synchronize()
    assert torch.equal(dst, src)
    assert V.voc_dbg_copy(dst, src, 10, s) == V.VOC_INVALID_PARAMS


def test_profile_select_times_only_selected_kinds(weights):
    ctx = V.open_context(CFG, weights)
    try:
        x = to_dev(I.make_latent(CFG, batch=2, frames=20))
        V.decode(ctx, x)
        convt = V.KERNEL_KINDS.index("convt")
        assert V.vocoder_profile_select(ctx, 1 << len(V.KERNEL_KINDS)) == V.VOC_INVALID_PARAMS
        V.check(V.vocoder_profile_reset(ctx))
        V.check(V.vocoder_profile_select(ctx, 1 << convt))
        V.check(V.vocoder_profile_enable(ctx, True))
        V.decode(ctx, x)
        V.check(V.vocoder_profile_enable(ctx, False))
        V.check(V.vocoder_profile_select(ctx, 0))
        for k, n in enumerate(V.KERNEL_KINDS):
            st, s = V.vocoder_profile_read(ctx, k)
            assert st == V.VOC_OK
            if n == "convt":
                assert s["launches"] == 4 and s["ms"] > 0
            elif n in ("conv_in", "head", "import"):
                assert s["launches"] == 1 and s["ms"] == 0 and (n == "import" or s["flops"] > 0)
    finally:
        V.vocoder_destroy(ctx)


def test_measured_peaks_are_plausible():
    """voc_dbg_peak: a copy and the matrix-core loops land below the published
    peaks (8 TB/s, 157.3 and 2500 TFLOP/s) and well above nothing; bad
    arguments are rejected."""
    st, gbs = V.voc_dbg_peak(0, 64 << 20)
    assert st == V.VOC_OK and 500 < gbs < 8000, gbs
    st, f32 = V.voc_dbg_peak(1, 200)
    assert st == V.VOC_OK and 20 < f32 < 157.3, f32
    st, bf16 = V.voc_dbg_peak(2, 2000)
    assert st == V.VOC_OK and 200 < bf16 < 2500, bf16
    for what, n, lo, hi in ((3, 100, 20, 157.3), (4, 1000, 200, 2500)):
        st, v = V.voc_dbg_peak(what, n)
        assert st == V.VOC_OK and lo < v < hi, (what, v)
    print(f"copy {gbs:.0f} GB/s, fp32 MFMA {f32:.1f} TFLOP/s, bf16 MFMA {bf16:.0f} TFLOP/s")
    assert V.voc_dbg_peak(0, 100)[0] == V.VOC_INVALID_PARAMS
    assert V.voc_dbg_peak(5, 100)[0] == V.VOC_INVALID_PARAMS
    assert V.voc_dbg_peak(1, 0)[0] == V.VOC_INVALID_PARAMS
