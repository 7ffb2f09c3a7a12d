"""The library's host code under AddressSanitizer and UBSan, on the CPU: a seeded
byte-mutation fuzz of the stats-file parser (the code that reads untrusted file
bytes) and the C ABI's argument validation (tests/asan_host_driver.cpp).  The
sanitizers instrument the host code only (each -fsanitize= follows -Xarch_host);
no GPU is used."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "key_importance_scoring_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("asan") / "asan_host_driver")
    cmd = [HIPCC, "-std=c++17", "--offload-arch=gfx950", "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "tria_kernels.hip"), os.path.join(CSRC, "tria_abi.cpp"),
           os.path.join(CSRC, "tria_stats.cpp"), os.path.join(HERE, "asan_host_driver.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


@pytest.mark.parametrize("seed", [1, 2])
def test_host_code_under_sanitizers(driver, seed):
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([driver, str(seed), "20000"], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert r.stdout.strip().endswith("ok"), r.stdout
