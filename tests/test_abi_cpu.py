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
    dict(af_snake=1, causal=1), dict(af_snake=1, enc_width=(0, 64)),
])
def test_invalid_configs_rejected_before_any_device_call(kw):
    c = _bad(**kw)
    assert V.voc_config_validate(c) == V.VOC_INVALID_PARAMS
    st, ctx = V.vocoder_create(c, 0)
    assert st == V.VOC_INVALID_PARAMS and not ctx.value
    assert V.vocoder_last_error(None)


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
