"""TriAttention KV-cache pruning pass (score -> select -> compact) on MI355X.

The compute lives in libtria.so (C ABI: include/tria.h, gfx950 HIP kernels under
csrc/).  This package holds its ctypes binding (``_lib``), the seeded synthetic
workloads (``synth``) and a torch-backed device harness (``device``).
"""
from ._lib import (TriaError, TriaKvView, TriaParams, load, make_params, make_view, tria_compact,  # noqa: F401
                   tria_device_flags, tria_score, tria_select, tria_timing_enable, tria_timing_read,
                   tria_workspace_size)
