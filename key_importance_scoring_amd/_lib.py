"""ctypes binding of libtria.so (include/tria.h).  Argument marshalling only.

Every function has the name and argument order of its C entry point.  Device
buffers may be passed as torch tensors (their ``data_ptr()`` is used) or as raw
integer addresses; ``stream`` is a HIP stream handle (an int; 0 = null stream)
or a ``torch.cuda.Stream``.  A non-OK status raises ``TriaError``.  The library
must have been built (``python -m key_importance_scoring_amd.build``): there is
no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtria.so")

TRIA_OK, TRIA_EINVAL, TRIA_ESHAPE, TRIA_EBUDGET, TRIA_EOVERLAP, TRIA_EWORKSPACE, TRIA_ELAUNCH = range(7)
PAIR_NEOX, PAIR_INTERLEAVED = 0, 1
AGG_MEAN, AGG_MAX = 0, 1
OFFSETS_MEAN, OFFSETS_MAX = 0, 1
FLAG_LEN, FLAG_LAYER, FLAG_BUDGET, FLAG_BLOCK, FLAG_INDEX, FLAG_BMAX, FLAG_SYNC = 1, 2, 4, 8, 16, 32, 64

EXPORTS = ("tria_workspace_size", "tria_score", "tria_select", "tria_compact", "tria_device_flags",
           "tria_strerror", "tria_last_error", "tria_timing_enable", "tria_timing_read", "tria_kernel_name",
           "tria_score_max_workgroups", "tria_score_wait_polls", "tria_log", "tria_select_strategy",
           "tria_calibrate_workspace_size",
           "tria_calibrate", "tria_compact_inplace", "tria_append", "tria_stats_parse", "tria_stats_encode",
           "tria_stats_band_mask", "tria_stats_layer_budgets", "tria_pass_noalloc")


class TriaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"tria status {status}: {message}")
        self.status = status


class TriaParams(ctypes.Structure):
    _fields_ = [("head_dim", c_int32), ("n_kv_heads", c_int32), ("group", c_int32), ("n_layers", c_int32),
                ("pairing", c_int32), ("agg", c_int32), ("rope_base", c_double),
                ("offsets", POINTER(c_int64)), ("n_offsets", c_int32), ("sink", c_int32), ("window", c_int32),
                ("offset_reduce", c_int32)]


class TriaKvView(ctypes.Structure):
    _fields_ = [("base", c_void_p), ("stride_unit", c_int64), ("stride_head", c_int64), ("stride_slot", c_int64),
                ("block_table", c_void_p), ("block_size", c_int32), ("max_blocks", c_int32),
                ("n_pool_blocks", c_int64)]


class TriaStatsInfo(ctypes.Structure):
    _fields_ = [("version", ctypes.c_uint32), ("n_layers", ctypes.c_uint32), ("n_heads", ctypes.c_uint32),
                ("n_kv_heads", ctypes.c_uint32), ("fc", ctypes.c_uint32), ("head_dim", ctypes.c_uint32),
                ("has_budget_scales", c_int32), ("mrl_present", c_int32)]


_lib = None


def load() -> ctypes.CDLL:
    """Load libtria.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m key_importance_scoring_amd.build`")
    # torch ships its own HIP runtime: loaded first, it is the one the library binds
    # to; loaded after, a second runtime would not know torch's device memory
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    lib.tria_workspace_size.restype = c_size_t
    lib.tria_workspace_size.argtypes = [POINTER(TriaParams), c_int32, c_int32]
    lib.tria_score.restype = c_int32
    lib.tria_score.argtypes = [POINTER(TriaParams), POINTER(TriaKvView), c_int32, c_int32,
                               c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                               c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.tria_select.restype = c_int32
    lib.tria_select.argtypes = [POINTER(TriaParams), c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.tria_compact.restype = c_int32
    lib.tria_compact.argtypes = [POINTER(TriaParams), POINTER(TriaKvView), POINTER(TriaKvView), c_void_p, c_int32,
                                 c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                 POINTER(TriaKvView), POINTER(TriaKvView), c_void_p, c_void_p]
    lib.tria_device_flags.restype = c_int32
    lib.tria_device_flags.argtypes = [c_void_p, POINTER(c_int32), c_void_p]
    lib.tria_strerror.restype = c_char_p
    lib.tria_strerror.argtypes = [c_int32]
    lib.tria_last_error.restype = c_char_p
    lib.tria_last_error.argtypes = []
    lib.tria_timing_enable.restype = c_int32
    lib.tria_timing_enable.argtypes = [c_int32]
    lib.tria_timing_read.restype = c_int32
    lib.tria_timing_read.argtypes = [POINTER(c_double), POINTER(c_int64), c_int32]
    lib.tria_kernel_name.restype = c_char_p
    lib.tria_kernel_name.argtypes = [c_int32]
    lib.tria_score_max_workgroups.restype = c_int32
    lib.tria_score_max_workgroups.argtypes = [c_int32]
    lib.tria_score_wait_polls.restype = c_int32
    lib.tria_score_wait_polls.argtypes = [c_int32]
    lib.tria_log.restype = c_int32
    lib.tria_log.argtypes = [c_int32]
    lib.tria_select_strategy.restype = c_int32
    lib.tria_select_strategy.argtypes = [c_int32]
    lib.tria_calibrate_workspace_size.restype = c_size_t
    lib.tria_calibrate_workspace_size.argtypes = [POINTER(TriaParams), c_int32]
    lib.tria_calibrate.restype = c_int32
    lib.tria_calibrate.argtypes = [POINTER(TriaParams), c_void_p, c_int64, c_int64, c_int64, c_int32,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.tria_compact_inplace.restype = c_int32
    lib.tria_compact_inplace.argtypes = [POINTER(TriaParams), POINTER(TriaKvView), POINTER(TriaKvView), c_void_p,
                                         c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p]
    lib.tria_append.restype = c_int32
    lib.tria_append.argtypes = [POINTER(TriaParams), POINTER(TriaKvView), POINTER(TriaKvView), c_void_p, c_int32,
                                c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                c_void_p]
    lib.tria_pass_noalloc.restype = c_int32
    lib.tria_pass_noalloc.argtypes = [POINTER(TriaParams), POINTER(TriaKvView), POINTER(TriaKvView), c_int32, c_int32,
                                      c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_int32, c_void_p, c_void_p, c_void_p, POINTER(TriaKvView),
                                      POINTER(TriaKvView), c_void_p, c_void_p, c_void_p]
    lib.tria_stats_parse.restype = c_int32
    lib.tria_stats_parse.argtypes = [c_void_p, c_size_t, POINTER(TriaStatsInfo), c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p]
    lib.tria_stats_encode.restype = c_size_t
    lib.tria_stats_encode.argtypes = [POINTER(TriaStatsInfo), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_size_t]
    lib.tria_stats_band_mask.restype = c_int32
    lib.tria_stats_band_mask.argtypes = [c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p]
    lib.tria_stats_layer_budgets.restype = c_int32
    lib.tria_stats_layer_budgets.argtypes = [c_int32, c_void_p, c_int32, c_void_p, c_int32, c_void_p]
    _lib = lib
    return lib


# ----------------------------------------------------------------------------- marshalling helpers

def ptr(x) -> int | None:
    """Device address of a tensor (or an int address); None stays NULL."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def stream_handle(stream) -> int | None:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_params(head_dim: int, n_kv_heads: int, group: int, n_layers: int, pairing: int, agg: int,
                rope_base: float, offsets, sink: int, window: int, offset_reduce: int = OFFSETS_MEAN) -> TriaParams:
    """A TriaParams; the offsets array is kept alive on the returned object."""
    arr = (c_int64 * len(offsets))(*[int(o) for o in offsets])
    p = TriaParams(head_dim, n_kv_heads, group, n_layers, pairing, agg, float(rope_base),
                   ctypes.cast(arr, POINTER(c_int64)), len(offsets), sink, window, offset_reduce)
    p._offsets_keepalive = arr
    return p


def make_view(base, stride_unit: int, stride_head: int, stride_slot: int, block_table=None,
              block_size: int = 0, max_blocks: int = 0, n_pool_blocks: int = 0) -> TriaKvView:
    return TriaKvView(ptr(base), stride_unit, stride_head, stride_slot, ptr(block_table),
                      block_size, max_blocks, n_pool_blocks)


def _check(status: int) -> None:
    if status != TRIA_OK:
        lib = load()
        msg = lib.tria_last_error().decode(errors="replace")
        raise TriaError(status, f"{lib.tria_strerror(status).decode()}: {msg}")


# ----------------------------------------------------------------------------- entry points

def tria_workspace_size(p: TriaParams, n_units: int, n_max: int) -> int:
    return int(load().tria_workspace_size(ctypes.byref(p), n_units, n_max))


def tria_score(p: TriaParams, k: TriaKvView, n_units: int, n_max: int, len_, unit_layer, q_pos,
               q_mean_re, q_mean_im, q_abs_mean, raw, agg, ws, ws_bytes: int, stream=None) -> None:
    _check(load().tria_score(ctypes.byref(p), ctypes.byref(k), n_units, n_max, ptr(len_), ptr(unit_layer),
                             ptr(q_pos), ptr(q_mean_re), ptr(q_mean_im), ptr(q_abs_mean), ptr(raw), ptr(agg),
                             ptr(ws), ws_bytes, stream_handle(stream)))


def tria_select(p: TriaParams, n_units: int, n_max: int, b_max: int, len_, budget, agg, idx, cnt,
                ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check(load().tria_select(ctypes.byref(p), n_units, n_max, b_max, ptr(len_), ptr(budget), ptr(agg),
                              ptr(idx), ptr(cnt), ptr(ws), ws_bytes, stream_handle(stream)))


def tria_compact(p: TriaParams, k_src: TriaKvView, v_src: TriaKvView, pos_src, pos_heads: int, n_units: int,
                 n_max: int, b_max: int, len_, idx, cnt, k_dst: TriaKvView, v_dst: TriaKvView, pos_dst,
                 stream=None) -> None:
    _check(load().tria_compact(ctypes.byref(p), ctypes.byref(k_src), ctypes.byref(v_src), ptr(pos_src), pos_heads,
                               n_units, n_max, b_max, ptr(len_), ptr(idx), ptr(cnt), ctypes.byref(k_dst),
                               ctypes.byref(v_dst), ptr(pos_dst), stream_handle(stream)))


def tria_calibrate_workspace_size(p: TriaParams, n_tokens: int) -> int:
    return int(load().tria_calibrate_workspace_size(ctypes.byref(p), n_tokens))


def tria_calibrate(p: TriaParams, q, stride_layer: int, stride_head: int, stride_token: int, n_tokens: int,
                   q_mean_re, q_mean_im, q_abs_mean, r, mrl, ws, ws_bytes: int, stream=None) -> None:
    _check(load().tria_calibrate(ctypes.byref(p), ptr(q), stride_layer, stride_head, stride_token, n_tokens,
                                 ptr(q_mean_re), ptr(q_mean_im), ptr(q_abs_mean), ptr(r), ptr(mrl), ptr(ws),
                                 ws_bytes, stream_handle(stream)))


def tria_compact_inplace(p: TriaParams, k: TriaKvView, v: TriaKvView, pos, n_units: int, n_max: int, b_max: int,
                         len_, idx, cnt, ws, stream=None) -> None:
    _check(load().tria_compact_inplace(ctypes.byref(p), ctypes.byref(k), ctypes.byref(v), ptr(pos), n_units, n_max,
                                       b_max, ptr(len_), ptr(idx), ptr(cnt), ptr(ws), stream_handle(stream)))


def tria_append(p: TriaParams, k: TriaKvView, v: TriaKvView, pos, n_units: int, n_max: int, len_, q_pos,
                t_new: int, k_new, v_new, pos_new, ws, stream=None) -> None:
    _check(load().tria_append(ctypes.byref(p), ctypes.byref(k), ctypes.byref(v), ptr(pos), n_units, n_max, ptr(len_),
                              ptr(q_pos), t_new, ptr(k_new), ptr(v_new), ptr(pos_new), ptr(ws),
                              stream_handle(stream)))


def tria_pass_noalloc(p: TriaParams, k: TriaKvView, v: TriaKvView, n_units: int, n_max: int, b_max: int, len_,
                      unit_layer, q_pos, budget, q_mean_re, q_mean_im, q_abs_mean, pos_src, pos_heads: int, agg, idx,
                      cnt, k_dst: TriaKvView, v_dst: TriaKvView, pos_dst, flags=None, stream=None) -> None:
    _check(load().tria_pass_noalloc(ctypes.byref(p), ctypes.byref(k), ctypes.byref(v), n_units, n_max, b_max,
                                    ptr(len_), ptr(unit_layer), ptr(q_pos), ptr(budget), ptr(q_mean_re),
                                    ptr(q_mean_im), ptr(q_abs_mean), ptr(pos_src), pos_heads, ptr(agg), ptr(idx),
                                    ptr(cnt), ctypes.byref(k_dst), ctypes.byref(v_dst), ptr(pos_dst), ptr(flags),
                                    stream_handle(stream)))


def tria_device_flags(ws, stream=None) -> int:
    out = c_int32(0)
    _check(load().tria_device_flags(ptr(ws), ctypes.byref(out), stream_handle(stream)))
    return int(out.value)


SELECT_AUTO, SELECT_PER_GROUP, SELECT_TILED = range(3)


def tria_select_strategy(strategy: int) -> int:
    """Sets tria_select's work distribution (SELECT_*); returns the previous one."""
    return int(load().tria_select_strategy(int(strategy)))


def tria_score_max_workgroups(cap: int) -> int:
    """Caps tria_score's persistent grid (0: device capacity); returns the previous cap."""
    return int(load().tria_score_max_workgroups(int(cap)))


def tria_score_wait_polls(polls: int) -> int:
    """Sets tria_score's bounded wait for a group's moments (< 0: compute them directly
    every time); returns the previous value."""
    return int(load().tria_score_wait_polls(int(polls)))


def tria_log(on: int) -> int:
    """The host decision log on stderr (1 on, 0 off, < 0 query); returns the previous state."""
    return int(load().tria_log(int(on)))


def tria_timing_enable(on: bool) -> int:
    return int(load().tria_timing_enable(int(bool(on))))


def tria_timing_read() -> dict:
    """{kernel name: (summed ms, launches)} since the previous read."""
    lib = load()
    n = 16
    ms = (c_double * n)()
    cnt = (c_int64 * n)()
    k = int(lib.tria_timing_read(ms, cnt, n))
    return {lib.tria_kernel_name(i).decode(): (ms[i], int(cnt[i])) for i in range(k)}


# ----------------------------------------------------------------------------- statistics files (host memory)

def _host_f32(a, shape=None):
    """A C-contiguous float32 numpy array (the caller's own when it already is one)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if shape is not None and a.shape != tuple(shape):
        a = a.reshape(shape)
    return a


def _np_ptr(a) -> int | None:
    return None if a is None else a.ctypes.data


def tria_stats_parse(data: bytes):
    """(info, q_mean_re, q_mean_im, q_abs_mean, mrl, layer_budget_scales): the
    statistics as float32 [n_layers][n_heads][fc], the scales as [n_layers]."""
    lib = load()
    buf = ctypes.create_string_buffer(bytes(data), len(data) + 1)     # never NULL, also for b""
    info = TriaStatsInfo()
    # first call: the header only (NULL outputs)
    _check(lib.tria_stats_parse(buf, len(data), ctypes.byref(info), None, None, None, None, None))
    shape = (info.n_layers, info.n_heads, info.fc)
    re, im, ab, mrl = (np.empty(shape, np.float32) for _ in range(4))
    scales = np.empty(info.n_layers, np.float32)
    _check(lib.tria_stats_parse(buf, len(data), ctypes.byref(info), _np_ptr(re), _np_ptr(im), _np_ptr(ab),
                                _np_ptr(mrl), _np_ptr(scales)))
    return info, re, im, ab, mrl, scales


def tria_stats_encode(version: int, n_kv_heads: int, q_mean_re, q_mean_im, q_abs_mean, mrl=None,
                      layer_budget_scales=None) -> bytes:
    """A stats file of the given version from float32 [n_layers][n_heads][fc] arrays."""
    re = _host_f32(q_mean_re)
    n_layers, n_heads, fc = re.shape
    im = _host_f32(q_mean_im, re.shape)
    ab = _host_f32(q_abs_mean, re.shape)
    mr = None if mrl is None else _host_f32(mrl, re.shape)
    sc = None if layer_budget_scales is None else _host_f32(layer_budget_scales, (n_layers,))
    info = TriaStatsInfo(version, n_layers, n_heads, n_kv_heads, fc, 2 * fc, int(sc is not None), int(version >= 2))
    lib = load()
    need = int(lib.tria_stats_encode(ctypes.byref(info), _np_ptr(re), _np_ptr(im), _np_ptr(ab), _np_ptr(mr),
                                     _np_ptr(sc), None, 0))
    if need == 0:
        raise TriaError(TRIA_EINVAL, "invalid stats header or arrays")
    out = np.empty(need, np.uint8)
    got = int(lib.tria_stats_encode(ctypes.byref(info), _np_ptr(re), _np_ptr(im), _np_ptr(ab), _np_ptr(mr),
                                    _np_ptr(sc), _np_ptr(out), need))
    assert got == need
    return out.tobytes()


def tria_stats_band_mask(mask, q_mean_re, q_mean_im, q_abs_mean) -> None:
    """In place on C-contiguous float32 arrays [..][fc]; mask is [fc]."""
    for a in (q_mean_re, q_mean_im, q_abs_mean):
        if not (isinstance(a, np.ndarray) and a.dtype == np.float32 and a.flags.c_contiguous and a.flags.writeable):
            raise TypeError("statistics must be writable C-contiguous float32 numpy arrays")
        if a.shape != q_mean_re.shape:
            raise ValueError("statistics arrays differ in shape")
    fc = q_mean_re.shape[-1]
    m = _host_f32(mask)
    if m.shape != (fc,):
        raise ValueError(f"mask has shape {m.shape}, expected ({fc},)")
    _check(load().tria_stats_band_mask(q_mean_re.size // fc, fc, _np_ptr(m), _np_ptr(q_mean_re),
                                       _np_ptr(q_mean_im), _np_ptr(q_abs_mean)))


def tria_stats_layer_budgets(unit_layer, layer_budget_scales, budget: int):
    """int32 [n_units] per-unit budgets for tria_select."""
    ul = np.ascontiguousarray(unit_layer, dtype=np.int32)
    sc = _host_f32(layer_budget_scales)
    out = np.empty(ul.size, np.int32)
    _check(load().tria_stats_layer_budgets(ul.size, _np_ptr(ul), sc.size, _np_ptr(sc), int(budget), _np_ptr(out)))
    return out
