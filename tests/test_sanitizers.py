"""CPU sanitizer builds.

* The oracle: oracle.c built with AddressSanitizer and UndefinedBehavior-
  Sanitizer (gcc), loaded by a child Python with the ASan runtime
  preloaded, runs every oracle pin; a copy with one out-of-bounds read
  planted must be caught.
* The library's host-only code (dac_vocoder_decoding_amd/csrc/
  host_config.cpp: configuration validation, exact halos, the GEMM plane
  limit, window bookkeeping, the checkpoint tensor table, the low-pass
  design) built with g++ under the same sanitizers, driven by
  tests/host_checks.cpp through the host-only C entry points and the
  helpers behind them.
No device code is built or run here.
"""
import os
import shutil
import subprocess
import sys

import pytest

from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
REPORT = ("AddressSanitizer", "runtime error:")


def _libasan():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not p or not os.path.exists(p):
        pytest.skip("gcc's ASan runtime is not installed")
    return p


def _build_oracle(src, out_dir):
    os.makedirs(out_dir, exist_ok=True)
    for prec in ("f64", "f32"):
        O.compile_library(src, os.path.join(out_dir, f"liboracle_{prec}.so"), prec, extra=SAN)


def _run_pins(libdir, *pytest_args):
    env = dict(os.environ, LD_PRELOAD=_libasan(), ASAN_OPTIONS="detect_leaks=0",
               VOC_ORACLE_LIBDIR=str(libdir), PYTHONPATH=ROOT)
    # --capture=sys: a sanitizer report goes to file descriptor 2 and must not
    # vanish into pytest's fd capture when the report ends the process.
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-q",
           "-p", "no:cacheprovider", "--capture=sys", *pytest_args]
    return subprocess.run(cmd, capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)


@pytest.mark.slow
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    _build_oracle(os.path.join(ROOT, "oracle", "oracle.c"), tmp_path / "san")
    nm = subprocess.run(["nm", "-D", str(tmp_path / "san" / "liboracle_f64.so")], capture_output=True,
                        text=True).stdout
    assert "__asan_" in nm and "__ubsan_" in nm          # the instrumented build is the one loaded
    r = _run_pins(tmp_path / "san")
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert not any(k in out for k in REPORT), out[-4000:]
    assert " passed" in out


def test_planted_out_of_bounds_read_is_caught(tmp_path):
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    good = "        const REAL s = SIN(a * xr[t]);"
    assert good in src
    bad = src.replace(good, "        const REAL s = SIN(a * xr[t + T]);")   # reads one row past the end
    p = tmp_path / "oracle_oob.c"
    p.write_text(bad)
    _build_oracle(str(p), tmp_path / "oob")
    r = _run_pins(tmp_path / "oob", "-x", "-k", "snake")
    out = r.stdout + r.stderr
    assert r.returncode != 0 and "AddressSanitizer" in out, out[-3000:]


def test_host_code_under_asan_and_ubsan(tmp_path):
    if not shutil.which("g++"):
        pytest.skip("g++ is not installed")
    exe = tmp_path / "host_checks"
    subprocess.run(["g++", "-std=c++17", "-O1", *SAN, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "dac_vocoder_decoding_amd", "csrc", "host_config.cpp"),
                    os.path.join(ROOT, "tests", "host_checks.cpp"), "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "host checks ok" in out and not any(k in out for k in REPORT), out[-4000:]
