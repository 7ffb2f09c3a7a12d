"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments
on the host before launching anything.

These tests run without a GPU.  Every call below either fails host validation or
has zero units, so no HIP call is made; the device addresses are fake and must
never reach a kernel (a call that passes validation here would launch on them).
"""
import ctypes
import os
import re

import pytest

import key_importance_scoring_amd as kis
from key_importance_scoring_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tria.h")

# fake, never-dereferenced device addresses (16-byte aligned)
A = 0x7F0000000000
WS = 0x7F1000000000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tria_[a-z_]+)\s*\(", src)))


def _params(**kw):
    base = dict(head_dim=128, n_kv_heads=8, group=4, n_layers=2, pairing=L.PAIR_NEOX, agg=L.AGG_MAX,
                rope_base=1e6, offsets=[2 ** i for i in range(17)], sink=4, window=128)
    base.update(kw)
    return L.make_params(**base)


def _view(base=A, **kw):
    d = dict(stride_unit=8 * 4096 * 128, stride_head=4096 * 128, stride_slot=128)
    d.update(kw)
    return L.make_view(base, **d)


def _score(p=None, k=None, n_units=2, n_max=4096, ws_bytes=None, raw=None, **kw):
    p = p or _params()
    k = k or _view()
    if ws_bytes is None:
        ws_bytes = L.tria_workspace_size(p, n_units, n_max)
    args = dict(len_=A, unit_layer=A, q_pos=A, q_mean_re=A, q_mean_im=A, q_abs_mean=A, raw=raw, agg=A, ws=WS)
    args.update(kw)
    L.tria_score(p, k, n_units, n_max, args["len_"], args["unit_layer"], args["q_pos"], args["q_mean_re"],
                 args["q_mean_im"], args["q_abs_mean"], args["raw"], args["agg"], args["ws"], ws_bytes)


def _status(fn):
    with pytest.raises(kis.TriaError) as e:
        fn()
    return e.value.status


def test_library_exports_every_declared_symbol():
    lib = L.load()
    declared = _declared()
    assert set(declared) == set(L.EXPORTS), (declared, L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_strerror_and_kernel_names():
    lib = L.load()
    for s in range(7):
        assert lib.tria_strerror(s)
    assert lib.tria_strerror(99) == b"unknown status"
    names = [lib.tria_kernel_name(i) for i in range(5)]
    assert names == [b"k_coef", b"k_score", b"k_select", b"k_compact", b"k_calib"]
    assert lib.tria_kernel_name(5) == b""


def test_workspace_size_grows_with_the_problem():
    p = _params()
    a = L.tria_workspace_size(p, 2, 4096)
    # flag word + coefficients [U][Hq][d] + norm weights [U][Hq][d/2] + tile moments + counters
    assert a >= 256 + 2 * 32 * 128 * 4 + 2 * 32 * 64 * 4 + 2 * 32 * 2 * 3 * 8 + 2 * 8 * 4
    assert L.tria_workspace_size(p, 4, 4096) > a
    assert L.tria_workspace_size(p, 2, 8192) > a
    assert L.tria_workspace_size(_params(head_dim=96), 2, 4096) == 0
    assert L.tria_workspace_size(p, -1, 4096) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), L.TRIA_ESHAPE),
    (dict(head_dim=0), L.TRIA_ESHAPE),
    (dict(group=9), L.TRIA_ESHAPE),
    (dict(group=0), L.TRIA_ESHAPE),
    (dict(n_kv_heads=0), L.TRIA_ESHAPE),
    (dict(n_layers=0), L.TRIA_ESHAPE),
    (dict(pairing=2), L.TRIA_EINVAL),
    (dict(agg=5), L.TRIA_EINVAL),
    (dict(rope_base=1.0), L.TRIA_EINVAL),
    (dict(rope_base=float("nan")), L.TRIA_EINVAL),
    (dict(offsets=[1, -2]), L.TRIA_EINVAL),
    (dict(offsets=[1 << 41]), L.TRIA_EINVAL),
    (dict(offsets=list(range(300))), L.TRIA_EINVAL),
    (dict(sink=-1), L.TRIA_EINVAL),
    (dict(window=-1), L.TRIA_EINVAL),
])
def test_score_rejects_bad_params(kw, status):
    p = _params(**kw)
    assert _status(lambda: _score(p=p, ws_bytes=1 << 40)) == status


def test_score_rejects_bad_offset_reduce():
    assert _status(lambda: _score(p=_params(offset_reduce=2), ws_bytes=1 << 40)) == L.TRIA_EINVAL


def test_max_over_offsets_rejects_blocks_beyond_lds():
    # d 256, G 8, 17 offsets: 8 heads x 3 blocks x 8 KiB of staged operands do not fit
    p = _params(head_dim=256, group=8, offset_reduce=L.OFFSETS_MAX)
    k = _view(stride_unit=8 * 4096 * 256, stride_head=4096 * 256, stride_slot=256)
    assert _status(lambda: _score(p=p, k=k, ws_bytes=1 << 40)) == L.TRIA_ESHAPE


def test_max_over_offsets_needs_more_workspace():
    mean = L.tria_workspace_size(_params(), 2, 4096)
    mx = L.tria_workspace_size(_params(offset_reduce=L.OFFSETS_MAX), 2, 4096)
    # 2 units x 8 KV heads x 9 blocks (two offsets of the 4 heads each) x 4 chunks x 64 lanes x 16 B
    assert mx - mean >= 2 * 8 * 9 * 4 * 64 * 16


def test_score_rejects_empty_offsets():
    p = _params()
    p.n_offsets = 0
    assert _status(lambda: _score(p=p, ws_bytes=1 << 40)) == L.TRIA_EINVAL


@pytest.mark.parametrize("field", ["len_", "unit_layer", "q_pos", "q_mean_re", "q_mean_im", "q_abs_mean", "agg"])
def test_score_rejects_null_pointers(field):
    assert _status(lambda: _score(**{field: None})) == L.TRIA_EINVAL


def test_score_shape_and_workspace_checks():
    assert _status(lambda: _score(n_max=4100)) == L.TRIA_ESHAPE          # n_max % 16
    assert _status(lambda: _score(n_units=-1)) == L.TRIA_EINVAL
    assert _status(lambda: _score(k=_view(base=A + 8))) == L.TRIA_ESHAPE  # misaligned rows
    assert _status(lambda: _score(k=_view(stride_slot=100))) == L.TRIA_ESHAPE
    assert _status(lambda: _score(k=_view(base=None))) == L.TRIA_EINVAL
    assert _status(lambda: _score(agg=A + 4)) == L.TRIA_ESHAPE
    assert _status(lambda: _score(ws=None)) == L.TRIA_EWORKSPACE
    assert _status(lambda: _score(ws=WS + 64)) == L.TRIA_EWORKSPACE      # 256-byte alignment
    need = L.tria_workspace_size(_params(), 2, 4096)
    assert _status(lambda: _score(ws_bytes=need - 1)) == L.TRIA_EWORKSPACE
    # a paged view whose block table cannot cover n_max slots
    paged = _view(block_table=A, block_size=16, max_blocks=10, n_pool_blocks=100)
    assert _status(lambda: _score(k=paged)) == L.TRIA_ESHAPE
    paged0 = _view(block_table=A, block_size=0, max_blocks=300, n_pool_blocks=100)
    assert _status(lambda: _score(k=paged0)) == L.TRIA_ESHAPE


def test_zero_units_is_a_no_op():
    # returns OK without launching anything (no GPU here)
    _score(n_units=0)
    L.tria_select(_params(), 0, 4096, 16, A, A, A, A, A, WS, L.tria_workspace_size(_params(), 0, 4096))


def test_select_checks():
    p = _params()
    need = L.tria_workspace_size(p, 2, 4096)
    assert _status(lambda: L.tria_select(p, 2, 4096, 16, None, A, A, A, A, WS, need)) == L.TRIA_EINVAL
    assert _status(lambda: L.tria_select(p, 2, 4096, -1, A, A, A, A, A, WS, need)) == L.TRIA_EINVAL
    assert _status(lambda: L.tria_select(p, 2, 4096, 16, A, A, A, A, A, WS, 100)) == L.TRIA_EWORKSPACE
    assert _status(lambda: L.tria_select(p, 2, 4096, 16, A, A, A, A, A, None, 0)) == L.TRIA_EWORKSPACE
    assert _status(lambda: L.tria_select(p, 2, 4096, 16, A, A, A, A, A, WS + 64, need)) == L.TRIA_EWORKSPACE
    assert _status(lambda: L.tria_select(p, 2, 4100, 16, A, A, A, A, A, WS, need)) == L.TRIA_ESHAPE
    assert _status(lambda: L.tria_select(p, 2, 4096, 16, A, A, A + 4, A, A, WS, need)) == L.TRIA_ESHAPE
    assert _status(lambda: L.tria_select(_params(agg=3), 2, 4096, 16, A, A, A, A, A, WS, need)) == L.TRIA_EINVAL


def _compact(k_src, v_src, k_dst, v_dst, pos_src=None, pos_dst=None, pos_heads=1, n_units=2, n_max=4096, b_max=2048):
    L.tria_compact(_params(), k_src, v_src, pos_src, pos_heads, n_units, n_max, b_max, A, A, A, k_dst, v_dst, pos_dst)


def test_compact_rejects_overlap():
    src_bytes = 2 * 8 * 4096 * 128 * 2
    ks = _view(A)
    vs = _view(A + src_bytes)
    dst = lambda base: L.make_view(base, 8 * 2048 * 128, 2048 * 128, 128)
    free0 = A + 2 * src_bytes
    dst_bytes = 2 * 8 * 2048 * 128 * 2
    assert _status(lambda: _compact(ks, vs, dst(A + 4096), dst(free0))) == L.TRIA_EOVERLAP  # into K source
    assert _status(lambda: _compact(ks, vs, dst(free0), dst(A + src_bytes))) == L.TRIA_EOVERLAP
    assert _status(lambda: _compact(ks, vs, dst(free0), dst(free0 + 256))) == L.TRIA_EOVERLAP
    # positions
    p0 = free0 + 2 * dst_bytes
    assert _status(lambda: _compact(ks, vs, dst(free0), dst(free0 + dst_bytes), pos_src=p0, pos_dst=p0 + 64)) \
        == L.TRIA_EOVERLAP
    assert _status(lambda: _compact(ks, vs, dst(free0), dst(free0 + dst_bytes), pos_src=p0, pos_heads=3)) \
        == L.TRIA_ESHAPE


def test_compact_requires_views():
    ks = _view(A)
    with pytest.raises(Exception):
        L.tria_compact(_params(), ks, ks, None, 1, 2, 4096, 2048, A, A, A, None, ks, None)
    assert _status(lambda: _compact(ks, ks, _view(None), _view(A))) == L.TRIA_EINVAL


def test_last_error_names_the_problem():
    try:
        _score(n_max=4100)
    except kis.TriaError as e:
        assert "multiple of 16" in str(e)


def test_score_workgroup_cap_is_process_wide_and_returns_previous():
    prev = L.tria_score_max_workgroups(37)
    try:
        assert L.tria_score_max_workgroups(5) == 37
        assert L.tria_score_max_workgroups(-4) == 5     # negative means no cap
        assert L.tria_score_max_workgroups(0) == 0
    finally:
        L.tria_score_max_workgroups(prev)


def test_select_strategy_is_process_wide_and_returns_previous():
    prev = L.tria_select_strategy(L.SELECT_TILED)
    try:
        assert L.tria_select_strategy(L.SELECT_PER_GROUP) == L.SELECT_TILED
        assert L.tria_select_strategy(99) == L.SELECT_PER_GROUP     # unknown means automatic
        assert L.tria_select_strategy(L.SELECT_AUTO) == L.SELECT_AUTO
    finally:
        L.tria_select_strategy(prev)


def _calibrate(p=None, q=A, strides=(32 * 1024 * 128, 1024 * 128, 128), n_tokens=1024, ws=WS, ws_bytes=None,
               outs=(A, A, A), r=None, mrl=None):
    p = p or _params()
    if ws_bytes is None:
        ws_bytes = L.tria_calibrate_workspace_size(p, n_tokens)
    L.tria_calibrate(p, q, *strides, n_tokens, *outs, r, mrl, ws, ws_bytes)


def test_calibrate_workspace_size():
    p = _params()
    # [L][Hq][chunks of 1024 tokens][d/2][5] fp32 partial sums
    assert L.tria_calibrate_workspace_size(p, 4096) == 2 * 32 * 4 * 64 * 5 * 4
    assert L.tria_calibrate_workspace_size(p, 4097) == 2 * 32 * 5 * 64 * 5 * 4
    assert L.tria_calibrate_workspace_size(p, 1) == 2 * 32 * 1 * 64 * 5 * 4
    assert L.tria_calibrate_workspace_size(p, 0) == 0
    assert L.tria_calibrate_workspace_size(_params(head_dim=96), 1024) == 0


def test_calibrate_checks():
    # every call below fails validation before any launch
    assert _status(lambda: _calibrate(n_tokens=0, ws_bytes=1 << 30)) == L.TRIA_EINVAL
    assert _status(lambda: _calibrate(q=None)) == L.TRIA_EINVAL
    assert _status(lambda: _calibrate(outs=(A, None, A))) == L.TRIA_EINVAL
    assert _status(lambda: _calibrate(q=A + 8)) == L.TRIA_ESHAPE
    assert _status(lambda: _calibrate(strides=(8, 8, 12))) == L.TRIA_ESHAPE
    assert _status(lambda: _calibrate(strides=(8, -8, 16))) == L.TRIA_ESHAPE
    assert _status(lambda: _calibrate(ws=None)) == L.TRIA_EWORKSPACE
    assert _status(lambda: _calibrate(ws=WS + 64)) == L.TRIA_EWORKSPACE
    need = L.tria_calibrate_workspace_size(_params(), 1024)
    assert _status(lambda: _calibrate(ws_bytes=need - 1)) == L.TRIA_EWORKSPACE
    assert _status(lambda: _calibrate(p=_params(pairing=7), ws_bytes=1 << 30)) == L.TRIA_EINVAL
    # more (layer, query head) pairs than one launch dimension holds
    big = _params(n_layers=2100, n_kv_heads=8, group=4)
    assert _status(lambda: _calibrate(p=big, ws_bytes=1 << 40)) == L.TRIA_ESHAPE


def test_compact_inplace_checks():
    p = _params()
    k = _view(A)
    v = _view(A + 2 * 8 * 4096 * 128 * 2)
    call = lambda **kw: L.tria_compact_inplace(kw.get("p", p), kw.get("k", k), kw.get("v", v), None, kw.get("U", 2),
                                               4096, 2048, kw.get("len_", A), A, A, kw.get("ws", WS))
    assert _status(lambda: call(len_=None)) == L.TRIA_EINVAL
    assert _status(lambda: call(ws=None)) == L.TRIA_EWORKSPACE
    assert _status(lambda: call(p=_params(pairing=9))) == L.TRIA_EINVAL
    assert _status(lambda: call(k=_view(A + 8))) == L.TRIA_ESHAPE
    assert _status(lambda: call(v=_view(A + 4096))) == L.TRIA_EOVERLAP      # K and V overlap
    call(U=0)                                                                  # nothing to do


def test_append_checks():
    p = _params()
    k = _view(A)
    v = _view(A + 2 * 8 * 4096 * 128 * 2)
    call = lambda **kw: L.tria_append(p, k, v, None, 2, 4096, A, None, kw.get("t", 128), kw.get("kn", A), A, None,
                                      kw.get("ws", WS))
    assert _status(lambda: call(kn=None)) == L.TRIA_EINVAL
    assert _status(lambda: call(kn=A + 8)) == L.TRIA_ESHAPE
    assert _status(lambda: call(t=-1)) == L.TRIA_EINVAL
    assert _status(lambda: call(ws=None)) == L.TRIA_EWORKSPACE
    call(t=0)


def test_pass_noalloc_checks():
    """The allocation-free pass rejects a workspace beyond its 96 MiB array, and bad
    parameters, before any HIP call."""
    p = _params()
    k = _view()
    v = _view(A + 2 * 8 * 4096 * 128 * 2)
    kd = _view(A + 4 * 8 * 4096 * 128 * 2)
    vd = _view(A + 6 * 8 * 4096 * 128 * 2)

    def call(p=p, n_units=2, n_max=4096):
        L.tria_pass_noalloc(p, k, v, n_units, n_max, 2048, A, A, A, A, A, A, A, A, 1, A, A, A, kd, vd, A)

    assert _status(lambda: call(p=_params(pairing=5))) == L.TRIA_EINVAL
    assert _status(lambda: call(n_units=-1)) == L.TRIA_EINVAL
    # 300 units x 8 KV heads x 32768 slots need far more than 96 MiB of workspace
    assert L.tria_workspace_size(p, 300, 32768) > 96 << 20
    assert _status(lambda: call(n_units=300, n_max=32768)) == L.TRIA_EWORKSPACE
    assert "scratch holds" in L.load().tria_last_error().decode()


def test_log_switch_is_process_wide_and_returns_previous():
    prev = L.tria_log(-1)
    try:
        L.tria_log(1)
        assert L.tria_log(-1) == 1          # a negative value only queries
        assert L.tria_log(0) == 1
        assert L.tria_log(-1) == 0
    finally:
        L.tria_log(prev)


def test_log_reports_each_error_once_on_stderr(capfd):
    prev = L.tria_log(1)
    try:
        capfd.readouterr()
        assert _status(lambda: _score(n_max=4100)) == L.TRIA_ESHAPE
        err = capfd.readouterr().err
        lines = [l for l in err.splitlines() if l.startswith("[tria] ")]
        assert len(lines) == 1 and "error" in lines[0] and "multiple of 16" in lines[0], err
        L.tria_log(0)
        assert _status(lambda: _score(n_max=4100)) == L.TRIA_ESHAPE
        assert "[tria]" not in capfd.readouterr().err
    finally:
        L.tria_log(prev)


@pytest.mark.parametrize("value,on", [("1", True), ("0", False), ("", False)])
def test_log_follows_the_environment(value, on):
    import subprocess
    import sys
    code = ("import key_importance_scoring_amd as kis\n"
            "from key_importance_scoring_amd import _lib as L\n"
            "p = L.make_params(128, 8, 4, 2, L.PAIR_NEOX, L.AGG_MAX, 1e6, [1, 2], 0, 0)\n"
            "try:\n"
            "    L.tria_select(p, 1, 100, 8, 1, 1, 1, 1, 1, None, 0)\n"
            "except kis.TriaError:\n"
            "    pass\n")
    env = dict(os.environ, TRIA_LOG=value, PYTHONPATH=ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    assert ("[tria] error" in r.stderr) == on, r.stderr
