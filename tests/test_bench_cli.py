"""Host-side argument checks of bench.py (no GPU work happens before them)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_exact_options_refuse_other_paths():
    for extra in (("--mixed", "1"), ("--inference", "5")):
        r = _run("--exact", "1", *extra)
        assert r.returncode == 2, extra
        assert "exact options" in r.stderr


def test_mixed_path_refuses_the_inference_exponential():
    r = _run("--mixed", "1", "--inference", "5")
    assert r.returncode == 2
    assert "MXFP8 path only" in r.stderr
