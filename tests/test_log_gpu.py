"""The host decision log (TRIA_LOG, tria_log) on real passes: one line per call naming
the kernels and sizes the host chose, and nothing when it is off."""
import pytest
import torch

from key_importance_scoring_amd import _lib as L
from key_importance_scoring_amd import synth
from key_importance_scoring_amd.device import DeviceProblem

pytestmark = pytest.mark.gpu


def _run_logged(prob, capfd, strategy=L.SELECT_AUTO):
    prev_log = L.tria_log(1)
    prev_sel = L.tria_select_strategy(strategy)
    try:
        capfd.readouterr()
        prob.run()
        torch.cuda.synchronize()
        err = capfd.readouterr().err
    finally:
        L.tria_log(prev_log)
        L.tria_select_strategy(prev_sel)
    return [l for l in err.splitlines() if l.startswith("[tria] ")]


def test_log_names_each_decision(capfd):
    # 5000 keys (n_max 5008): three balanced score tiles of 1792 keys, three selection tiles
    cfg = synth.CONFIGS["qwen3_8b"].replace(name="log_dense", n_layers=2, n_kv=5000, budget=1000)
    print(f"[log] {cfg.name}", flush=True)
    prob = DeviceProblem(cfg)
    lines = _run_logged(prob, capfd)
    assert prob.flags() == 0
    score = [l for l in lines if l.startswith("[tria] score:")]
    select = [l for l in lines if l.startswith("[tria] select:")]
    compact = [l for l in lines if l.startswith("[tria] compact:")]
    assert len(score) == len(select) == len(compact) == 1, lines
    assert "k_score," in score[0] and "tiles of 1792 keys (3 per (unit, KV head), 48 in all)" in score[0], score
    assert "dense K" in score[0] and "NEOX" in score[0], score
    assert "k_sel_thresh" in select[0] and "3 selection tiles of 2048 slots" in select[0], select
    assert "k_compact_fast" in compact[0] and "dense -> dense" in compact[0], compact
    assert not any("error" in l for l in lines), lines
    # off again: silent
    capfd.readouterr()
    prob.run()
    torch.cuda.synchronize()
    assert "[tria]" not in capfd.readouterr().err


def test_log_per_group_selection_and_paged_views(capfd):
    cfg = synth.CONFIGS["batched_decode"].replace(name="log_paged", n_seqs=3, n_kv=4000, ragged_min=1000)
    print(f"[log] {cfg.name}", flush=True)
    prob = DeviceProblem(cfg)
    lines = _run_logged(prob, capfd, L.SELECT_PER_GROUP)
    assert prob.flags() == 0
    assert any(l.startswith("[tria] score:") and "paged K" in l for l in lines), lines
    assert any(l.startswith("[tria] select:") and "k_sel_group" in l for l in lines), lines
    assert any(l.startswith("[tria] compact:") and "paged -> paged" in l for l in lines), lines


def test_log_score_buffer_mode(capfd):
    # G = 8, the mean over offsets: a call whose 2048-key tiles all fit on the device
    # at once takes the single-buffer mode (8 KV heads x 3 tiles); Qwen3-8B's G = 4
    # keeps two buffers
    cfg = synth.CONFIGS["long_context"].replace(name="log_single", n_kv=6000, budget=600)
    print(f"[log] {cfg.name}", flush=True)
    prob = DeviceProblem(cfg)
    lines = _run_logged(prob, capfd)
    assert prob.flags() == 0
    score = [l for l in lines if l.startswith("[tria] score:")]
    assert len(score) == 1, lines
    assert "tiles of 2048 keys (3 per (unit, KV head), 24 in all), one score buffer" in score[0], score
    cfg = synth.CONFIGS["qwen3_8b"].replace(name="log_two", n_layers=1, n_kv=3000, budget=600)
    prob = DeviceProblem(cfg)
    lines = _run_logged(prob, capfd)
    assert any(l.startswith("[tria] score:") and "two score buffers" in l for l in lines), lines
