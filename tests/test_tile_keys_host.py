"""The score kernel's tile sizes, checked on the CPU over every n_max up to the
longest row the kernel takes (tests/tile_keys_check.cpp): multiples of 256 keys
within their caps, and the single-buffer mode's tiles never more per row than the
tiles the workspace's moment array is sized for."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "key_importance_scoring_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def test_tile_sizes(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path / "tile_keys_check")
    cmd = [HIPCC, "-std=c++17", "-O2", "--offload-arch=gfx950", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(HERE, "tile_keys_check.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    r = subprocess.run([out], capture_output=True, text=True, timeout=300, env=dict(os.environ, HIP_VISIBLE_DEVICES=""))
    assert r.returncode == 0, r.stdout[-2000:]
    assert r.stdout.strip().endswith("ok"), r.stdout
