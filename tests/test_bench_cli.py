"""bench.py's command line on the CPU: it measures one GPU only, so asking for more
exits with status 2 and says why, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _bench("--gpus", n, "--steps", "1", "--warmup", "0")
        assert r.returncode == 2, r.stderr
        assert f"--gpus {n} is not supported" in r.stderr
        assert r.stdout == ""        # no JSON line


def test_unknown_choice_is_an_argument_error():
    r = _bench("--offsets", "median")
    assert r.returncode == 2
    assert "invalid choice" in r.stderr
