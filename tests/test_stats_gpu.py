"""GPU parity of a pass driven by a loaded statistics file: the statistics of the
workload are written to a TRIA file, parsed back, band-masked and turned into
per-layer budgets by the library's host functions, and the HIP pass on those
statistics and budgets is compared with the fp64 oracle on the same (loaded,
masked) statistics and budgets.  The loader and the mask are pinned on the CPU
(test_stats.py); this checks that their outputs drive the device pass as the
statistics and budgets the oracle assumes, with masked-out bands (zero centres)
among them.
"""
import numpy as np
import pytest
import torch

from _parity import check_agg, check_compaction, check_kept, check_raw, log, oracle_head
from oracle import tria_oracle as o
from key_importance_scoring_amd import _lib as L
from key_importance_scoring_amd import synth
from key_importance_scoring_amd.device import DeviceProblem

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


@pytest.mark.parametrize("reduce", ["mean", "max"])
def test_loaded_masked_statistics_drive_the_pass(reduce):
    cfg = synth.CONFIGS["qwen3_8b"].replace(name=f"stats_{reduce}", n_layers=3, n_kv=3001, budget=1200,
                                            offset_reduce=reduce)
    F = cfg.head_dim // 2
    re, im, ab = synth.q_stats(cfg)
    scales = np.array([1.0, 0.6, 0.25], np.float32)
    data = L.tria_stats_encode(3, cfg.n_kv_heads, re, im, ab, None, scales)
    info, lre, lim, lab, _, lsc = L.tria_stats_parse(data)
    assert (info.n_layers, info.n_heads, info.fc) == (cfg.n_layers, cfg.n_q_heads, F)
    mask = np.ones(F, np.float32)
    mask[:6] = 0.0                                   # the fastest bands masked out
    mask[6:12] = 0.5
    L.tria_stats_band_mask(mask, lre, lim, lab)
    u = synth.units(cfg)
    budgets = L.tria_stats_layer_budgets(u.unit_layer, lsc, cfg.budget)
    assert set(budgets.tolist()) == {1200, 720, 300}
    log(f"[stats] {cfg.name}: units={cfg.n_units} budgets={sorted(set(budgets.tolist()))} reduce={reduce}")

    prob = DeviceProblem(cfg)
    dev = prob.q_re.device
    for t, a in ((prob.q_re, lre), (prob.q_im, lim), (prob.q_abs, lab)):
        t.copy_(torch.from_numpy(a).to(dev))
    prob.budget.copy_(torch.from_numpy(budgets).to(dev))
    prob.run()
    torch.cuda.synchronize()
    assert prob.flags() == 0

    mu = lre.astype(np.float64) + 1j * lim.astype(np.float64)
    absm = lab.astype(np.float64)
    form = "direct" if reduce == "max" else "folded"
    G = cfg.group
    cnt = prob.cnt.cpu().numpy()
    for unit in range(cfg.n_units):
        n = int(u.lengths[unit])
        B = int(budgets[unit])
        assert int(cnt[unit]) == min(B, n)
        for g in range(cfg.n_kv_heads):
            what = f"{cfg.name} unit {unit} kv {g}"
            o_raw, o_agg, _ = oracle_head(cfg, unit, g, form, mu, absm)
            o_kept = o.select(o_agg, B)
            if prob.raw is not None:
                check_raw(prob.raw[unit, g * G:(g + 1) * G, :n].cpu().numpy(), o_raw, what)
            check_agg(prob.agg[unit, g, :n].cpu().numpy(), o_agg, what)
            g_kept = prob.kept(unit, g)
            check_kept(g_kept, o_kept, o_agg, n, B, cfg.sink, cfg.window, what)
            check_compaction(prob, unit, g, g_kept, what)
