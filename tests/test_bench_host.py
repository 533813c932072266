"""Host-side contract of bench.py that needs no GPU: its options parse, and a
request for more than one GPU is refused with a message before any device
work starts."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_bench_help_parses():
    r = run_bench("--help")
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--only"):
        assert opt in r.stdout


def test_bench_refuses_more_than_one_gpu():
    r = run_bench("--gpus", "2", "--steps", "5", "--warmup", "1")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
