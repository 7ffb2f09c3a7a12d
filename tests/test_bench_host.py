"""bench.py's host-side parts without a GPU: the oracle CPU baseline over a process
pool (a short run on the tiny workload) and the read probe's argument checks (which
return before anything is launched)."""
import ctypes
import os

import pytest

import bench
from key_importance_scoring_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_cpu_baseline_pool_reports_both_forms():
    cfg = synth.CONFIGS["tiny"]
    r = bench.cpu_baseline(cfg, 0.2)
    assert r["kind"] == "oracle" and r["unit"] == "M keys/s"
    assert 1 <= r["cores"] <= 16
    assert set(r["forms"]) == {"folded", "direct"}
    for f in r["forms"].values():
        assert f["value"] > 0 and f["keys"] > 0 and f["pairs"] >= r["cores"]
    assert r["value"] == r["forms"]["folded"]["value"]


def test_cpu_baseline_maximum_over_offsets_has_the_direct_form_only():
    cfg = synth.CONFIGS["tiny"].replace(name="tiny_offsets_max", offset_reduce="max")
    r = bench.cpu_baseline(cfg, 0.1)
    assert set(r["forms"]) == {"direct"}
    assert "maximum over offsets" in r["sample"]


def _probe():
    path = os.path.join(ROOT, "key_importance_scoring_amd", "libtria_probe.so")
    if not os.path.exists(path):
        pytest.skip("libtria_probe.so is not built")
    lib = ctypes.CDLL(path)
    lib.tria_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.tria_probe_read.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("src,nbytes,tile,grid,sink", [
    (None, 1 << 20, 1 << 19, 512, 0x7F0000000000),              # no source
    (0x7F0000000000, 1 << 20, 1 << 19, 512, None),              # no sink
    (0x7F0000000000, (1 << 20) + 8, 1 << 19, 512, 0x7F1000000000),   # bytes not a multiple of 16
    (0x7F0000000000, 1 << 20, 100, 512, 0x7F1000000000),        # tile not a multiple of 16
    (0x7F0000000000, 1 << 20, 1 << 19, 0, 0x7F1000000000),      # empty grid
    (0x7F0000000008, 1 << 20, 1 << 19, 512, 0x7F1000000000),    # misaligned source
    (0x7F0000000000, 0, 1 << 19, 512, 0x7F1000000000),          # nothing to read
])
def test_read_probe_rejects_bad_arguments(src, nbytes, tile, grid, sink):
    assert _probe().tria_probe_read(src, nbytes, tile, grid, sink, None) == -1
