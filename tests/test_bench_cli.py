"""bench.py's argument handling on the CPU: runs above one GPU and two-term
operands on an fp32 workload are refused with a message and exit status 2,
before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_two_term_operands_need_a_bf16_workload():
    r = _bench("--config", "1", "--operand-terms", "2", "--no-cpu-baseline")
    assert r.returncode == 2
    assert "bf16" in r.stderr and r.stdout == ""
