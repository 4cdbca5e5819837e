"""CPU-side checks of the C ABI: the library loads and exports exactly what
include/vocoder.h declares, a plain C99 consumer compiles and runs its
validation paths, and the host-only entry points (config validation, hop,
exact halo) behave.  No kernel runs here."""
import ctypes
import os
import re
import subprocess

import pytest

from dac_vocoder_decoding_amd import inputs as I
from dac_vocoder_decoding_amd import vocoder as V

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vocoder.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:voc|vocoder)_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = V.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", V.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(names), exported ^ set(names)


def test_c99_consumer(tmp_path):
    exe = tmp_path / "abi_smoke"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "abi_c_smoke.c"),
                    V.LIB_PATH, f"-Wl,-rpath,{os.path.dirname(V.LIB_PATH)}", "-o", str(exe)],
                   check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    assert "abi ok" in res.stdout


@pytest.mark.parametrize("idx", sorted(I.CONFIGS))
def test_configs_validate(idx):
    cfg = V.config_from_dict(I.CONFIGS[idx])
    assert V.voc_config_validate(cfg) == V.VOC_OK
    assert V.voc_config_hop(cfg) == I.CONFIGS[idx]["hop"]


@pytest.mark.parametrize("idx,strides,halo", [(1, None, 10), (4, None, 10), (5, None, 10),
                                              (7, None, 20), (7, (8, 8, 4, 2), 19),
                                              (9, None, 30), (9, (8, 8, 4, 2), 20)])
def test_halo_matches_oracle_brute_force(idx, strides, halo):
    # The oracle's tiling pins show these halos reproduce the untiled decode
    # and one frame less does not (causal stacks: the left halo; alias-free
    # stacks: the structural reach a NaN marker shows); the library's
    # interval propagation must land on the same values.
    d = dict(I.CONFIGS[idx])
    if strides:
        d["strides"] = strides
        d["widths"] = d["widths"][:len(strides) + 1]
    assert V.voc_config_halo(V.config_from_dict(d)) == halo


def _bad(**kw):
    c = V.config_from_dict(I.CONFIGS[1])
    for k, v in kw.items():
        if isinstance(v, tuple):
            getattr(c, k)[v[0]] = v[1]
        else:
            setattr(c, k, v)
    return c


@pytest.mark.parametrize("kw", [
    dict(n_blocks=0), dict(n_blocks=9), dict(n_res=0), dict(in_kernel=5), dict(act=7),
    dict(dtype=3), dict(convt_crop=1), dict(tile_frames=-1), dict(latent_channels=60),
    dict(width=(2, 100)), dict(width=(4, 1024)), dict(stride=(0, 0)), dict(dilation=(1, 10)),
    dict(snake_log_params=2), dict(in_proj=-16), dict(in_proj=24), dict(in_proj=8208),
    dict(causal=2), dict(causal=-1), dict(af_snake=2), dict(out_channels=0), dict(out_channels=3),
    dict(convt_crop=2, causal=1), dict(convt_crop=-1),
    dict(af_snake=1, causal=1), dict(af_snake=1, enc_width=(0, 64)),
    dict(operand_terms=3), dict(operand_terms=-1), dict(operand_terms=2),  # the last: an fp32 config
    dict(operand_terms=2, dtype=1, af_snake=1),
    dict(operand_terms=2, dtype=1, in_proj=64), dict(operand_terms=2, dtype=1, enc_width=(0, 64)),
])
def test_invalid_configs_rejected_before_any_device_call(kw):
    c = _bad(**kw)
    assert V.voc_config_validate(c) == V.VOC_INVALID_PARAMS
    st, ctx = V.vocoder_create(c, 0)
    assert st == V.VOC_INVALID_PARAMS and not ctx.value
    assert V.vocoder_last_error(None)


def test_two_term_operands_validate_for_bf16_decoders():
    """operand_terms = 2 is a bf16 decoder option: accepted with dtype BF16
    (plain, tiled, stereo windows), 0 and 1 mean one term."""
    for terms in (0, 1):
        assert V.voc_config_validate(_bad(operand_terms=terms)) == V.VOC_OK
    for idx in (2, 4, 7):
        d = dict(I.CONFIGS[idx])
        d["operand_terms"] = 2
        assert V.voc_config_validate(V.config_from_dict(d)) == V.VOC_OK
        d["tile_frames"] = 128
        assert V.voc_config_validate(V.config_from_dict(d)) == V.VOC_OK


def test_causal_crop_named_explicitly():
    """convt_crop = 1 names the causal ConvTranspose1d crop; it is the crop a
    causal decoder takes anyway, so it validates exactly with causal = 1."""
    d = dict(I.CONFIGS[7])
    c = V.config_from_dict(d)
    assert c.causal == 1 and c.convt_crop == 0
    assert V.voc_config_validate(c) == V.VOC_OK
    c.convt_crop = 1
    assert V.voc_config_validate(c) == V.VOC_OK
    assert V.voc_config_hop(c) == V.voc_config_hop(V.config_from_dict(d))
    assert V.voc_config_halo(c) == V.voc_config_halo(V.config_from_dict(d))


def test_bf16_width_granularity():
    d = dict(I.CONFIGS[2])
    d["widths"] = (1024, 512, 256, 128, 48)   # 48 % 32 != 0
    assert V.voc_config_validate(V.config_from_dict(d)) == V.VOC_INVALID_PARAMS
    d["dtype"] = "f32"                          # 48 % 16 == 0
    assert V.voc_config_validate(V.config_from_dict(d)) == V.VOC_OK


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(V, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(V, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        V.lib()


def test_alias_free_snake_needs_a_plain_decoder():
    """The alias-free Snake is built for non-causal decoders without an
    encoder; the configurations that combine them are rejected on the host."""
    for idx, why in ((8, "decoder only"), (7, "non-causal")):
        c = V.config_from_dict(dict(I.CONFIGS[idx], af_snake=1))
        assert V.voc_config_validate(c) == V.VOC_INVALID_PARAMS
        st, ctx = V.vocoder_create(c, 0)
        assert st == V.VOC_INVALID_PARAMS and not ctx.value
        assert why in V.vocoder_last_error(None)
    assert V.voc_config_validate(V.config_from_dict(I.CONFIGS[9])) == V.VOC_OK


def _rate_max(d):
    """Largest input rate (frames per latent frame) among the decoder's GEMM
    launches: every ConvTranspose1d at its input rate, and the residual convs
    of the blocks whose units have no fused kernel (fp32: widths up to 128;
    bf16: 64, 96, 128, 192) at the block's output rate; alias-free decoders
    run every unit as a GEMM pair."""
    fused = {"f32": {16, 32, 64, 96, 128}, "bf16": {64, 96, 128, 192}}[d["dtype"]]
    rate, mx = 1, 1
    for b, s in enumerate(d["strides"]):
        mx = max(mx, rate)
        rate *= s
        if d.get("af_snake", 0) or d["widths"][b + 1] not in fused:
            mx = max(mx, rate)
    return mx


@pytest.mark.parametrize("idx", sorted(I.CONFIGS))
def test_max_frames_keeps_every_gemm_plane_below_4gib(idx):
    """The GEMMs address a 64-byte-per-frame channel plane with 32-bit byte
    offsets: the plane, the 54 context frames a stream carries and the 512
    rows a tile reads past its end must stay under 2^32 - 2^16 bytes.  The
    limit is set by the highest-rate GEMM layer."""
    d = I.CONFIGS[idx]
    m = V.voc_config_max_frames(V.config_from_dict(d))
    r = _rate_max(d)
    limit = (2 ** 32 - 2 ** 16) // 64 - 54 - 512
    assert m == limit // r, (m, r)
    assert (m * r + 54 + 512) * 64 <= 2 ** 32 - 2 ** 16
    assert ((m + 1) * r + 54 + 512) * 64 > 2 ** 32 - 2 ** 16


def test_max_frames_default_decoder():
    # widths 1024..64 fp32: units at 128 and 64 channels are fused, so the
    # last ConvTranspose1d (input rate 512 / 2 = 256) bounds the rows.
    c = V.voc_config_default()
    assert V.voc_config_max_frames(c) == ((2 ** 32 - 2 ** 16) // 64 - 566) // 256
    c.width[4] = 256       # the last block's units now run as GEMMs at rate 512
    c.width[3] = 256
    assert V.voc_config_max_frames(c) == ((2 ** 32 - 2 ** 16) // 64 - 566) // 512


def test_set_cancel_validates_arguments():
    assert V.lib().vocoder_set_cancel(None, V.CANCEL_FN(), None, 1) == V.VOC_INVALID_PARAMS


@pytest.mark.parametrize("shape,dim,want,ok", [
    ((2, 64, 9), 1, 64, True), ((2, 63, 9), 1, 64, False), ((3, 64, 9), 0, 2, False),
    ((2, 64), 1, 64, False), ((2, 128, 4), 1, 128, True)])
def test_binding_shape_check(shape, dim, want, ok):
    """The binding's helpers check the channel count (and a stream's row
    count) against the context before any call that would let the library
    read or write past the caller's buffers."""
    if ok:
        V.expect_dim("latent", shape, dim, want)
    else:
        with pytest.raises(ValueError):
            V.expect_dim("latent", shape, dim, want)
