"""GPU parity: the HIP pass (through the C ABI) against the fp64 oracle.

Small cases run every unit and KV head element by element; they span several
score tiles (2048 keys) with ragged tails, both pairings, head dims 64/128/256,
mean and max aggregation, paged caches and the degenerate budgets.  The full-size
workloads run in the same launch configuration as the benchmark and are checked
on every (unit, KV head) against the folded oracle (in a process pool over the
host cores), and on sampled pairs against the literal loop over the offsets.
"""
import re

import numpy as np
import pytest
import torch

from _parity import (check_agg, check_compaction, check_compaction_on_device, check_kept, check_raw,
                     check_unit, log, oracle_head, oracle_pairs)
from oracle import tria_oracle as o
from key_importance_scoring_amd import _lib as L
from key_importance_scoring_amd import synth
from key_importance_scoring_amd.device import DeviceProblem

pytestmark = pytest.mark.gpu

C = synth.CONFIGS
SMALL = {
    "tiny": C["tiny"],
    "q8_small": C["qwen3_8b"].replace(name="q8_small", n_layers=2, n_kv=5003, budget=1000),
    "q32_small": C["qwen3_32b"].replace(name="q32_small", n_layers=3, n_kv=4099, budget=1500, nonconc_frac=0.25),
    "bd_small": C["batched_decode"].replace(name="bd_small", n_seqs=6, n_kv=3000, ragged_min=300),
    "lc_small": C["long_context"].replace(name="lc_small", n_kv=6000, budget=600),
    "d256_neox": C["qwen3_8b"].replace(name="d256_neox", head_dim=256, n_layers=1, n_kv_heads=2, n_kv=2500,
                                       budget=700),
    "d256_inter": C["long_context"].replace(name="d256_inter", head_dim=256, n_kv_heads=2, group=3, n_kv=2100,
                                            budget=900),
    "d64_inter": C["tiny"].replace(name="d64_inter", pairing="interleaved", n_kv=3001, budget=1200, sink=3,
                                   agg="max"),
    # G > 4 on a dense cache at d = 256 and d = 64: the single-buffer score kernel
    "d256_g8": C["long_context"].replace(name="d256_g8", head_dim=256, n_kv_heads=2, n_kv=4500, budget=900,
                                         pairing="neox"),
    "d64_g6": C["tiny"].replace(name="d64_g6", group=6, n_kv=3333, budget=1100, agg="mean"),
    "g1_g7": C["qwen3_8b"].replace(name="g1", n_layers=1, n_kv_heads=3, group=1, n_kv=2300, budget=400),
    "g7": C["qwen3_8b"].replace(name="g7", n_layers=1, n_kv_heads=2, group=7, n_kv=2222, budget=800, agg="mean"),
    "keep_all": C["tiny"].replace(name="keep_all", n_kv=900, budget=5000),
    "all_protected": C["tiny"].replace(name="all_protected", n_kv=200, window=256, budget=300),
    "short_units": C["batched_decode"].replace(name="short_units", n_seqs=5, n_kv=40, ragged_min=1, window=8,
                                              sink=2, budget_frac=0.5),
    # scores whose mean is over 10^3 standard deviations: tightly concentrated keys,
    # query centres 10^-4 of E|q_f| (the norm term dominates the score); the moments and
    # the norm term's operands must keep the z-scores to the tolerance
    "concentrated": C["qwen3_8b"].replace(name="concentrated", n_layers=2, n_kv=5003, budget=1000,
                                          key_noise=0.002, mu_scale=1e-4),
    "concentrated_lc": C["long_context"].replace(name="concentrated_lc", n_kv=6000, budget=600, agg="mean",
                                                 key_noise=0.002, mu_scale=1e-4),
    # more units than the score kernel keeps lengths of in LDS: every tile is claimed
    "many_units": C["batched_decode"].replace(name="many_units", n_seqs=520, n_kv_heads=2, n_kv=2200,
                                             ragged_min=16, window=64, budget_frac=0.4),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _run(cfg, **kw):
    log(f"[parity] {cfg.name}: units={cfg.n_units} Hkv={cfg.n_kv_heads} G={cfg.group} d={cfg.head_dim} "
        f"n_kv={cfg.n_kv} pairing={cfg.pairing} paged={cfg.paged}")
    prob = DeviceProblem(cfg, **kw)
    prob.run()
    torch.cuda.synchronize()
    prob.check_guards()
    return prob


def _oracle_idx(prob, kept_by_unit):
    """An idx tensor holding the oracle's kept slots (the GPU's elsewhere)."""
    idx = prob.idx.clone()
    for unit, per_head in kept_by_unit.items():
        for g, kept in per_head.items():
            idx[unit, g, :kept.size] = torch.from_numpy(kept.astype(np.int32)).to(idx.device)
    return idx


def _check_oracle_compaction(prob, kept_by_unit):
    prob.compact(idx=_oracle_idx(prob, kept_by_unit))
    torch.cuda.synchronize()
    prob.check_guards()
    for unit, per_head in kept_by_unit.items():
        for g, kept in per_head.items():
            check_compaction(prob, unit, g, kept, f"{prob.cfg.name} unit {unit} kv {g} (oracle idx)")


def _expected_flags(cfg):
    """TRIA_FLAG_BUDGET is expected where a budget is below the protected slots of a
    unit that holds more keys than its budget."""
    u = synth.units(cfg)
    prot = np.minimum(u.lengths, cfg.sink + cfg.window)
    return L.FLAG_BUDGET if bool(((u.lengths > u.budget) & (u.budget < prot)).any()) else 0


@pytest.mark.parametrize("name", list(SMALL))
def test_small_parity(name):
    cfg = SMALL[name]
    prob = _run(cfg)
    assert prob.flags() == _expected_flags(cfg)
    form = "direct" if name == "tiny" else "folded"
    kept = {unit: check_unit(prob, unit, form=form) for unit in range(cfg.n_units)}
    _check_oracle_compaction(prob, kept)


# maximum over the offsets: every layout of the offset blocks (a shared block of each
# head's last offset, a padded last block per head, whole blocks only), both
# pairings, d 64 / 128 / 256, G 3 / 4 / 8, dense and paged
MAXO = {
    "q8_max": C["qwen3_8b"].replace(name="q8_max", n_layers=2, n_kv=5003, budget=1000, offset_reduce="max"),
    "lc_max": C["long_context"].replace(name="lc_max", n_kv=6000, budget=600, offset_reduce="max"),
    "bd_max": C["batched_decode"].replace(name="bd_max", n_seqs=6, n_kv=3000, ragged_min=300,
                                          offset_reduce="max"),
    "d256_max": C["qwen3_8b"].replace(name="d256_max", head_dim=256, n_layers=1, n_kv_heads=2, n_kv=2500,
                                      budget=700, offset_reduce="max"),
    "d64_max_3off": C["tiny"].replace(name="d64_max_3off", pairing="interleaved", n_kv=3001, budget=1200,
                                      offsets=(1, 2, 4), offset_reduce="max", agg="max"),
    "g3_max_9off": C["long_context"].replace(name="g3_max_9off", head_dim=128, n_kv_heads=2, group=3, n_kv=2100,
                                             budget=900, offsets=tuple(2 ** i for i in range(9)),
                                             offset_reduce="max"),
    "max_16off": C["qwen3_8b"].replace(name="max_16off", n_layers=1, n_kv_heads=2, n_kv=2222, budget=800,
                                       offsets=tuple(2 ** i for i in range(16)), offset_reduce="max"),
    "max_1off": C["tiny"].replace(name="max_1off", n_kv=1500, offsets=(64,), offset_reduce="max"),
    "g1_max": C["qwen3_8b"].replace(name="g1_max", n_layers=1, n_kv_heads=3, group=1, n_kv=2300, budget=400,
                                    offset_reduce="max"),
    "g7_max": C["qwen3_8b"].replace(name="g7_max", n_layers=1, n_kv_heads=2, group=7, n_kv=2222, budget=800,
                                    agg="mean", offset_reduce="max"),
    "concentrated_max": C["qwen3_8b"].replace(name="concentrated_max", n_layers=1, n_kv=3001, budget=700,
                                              key_noise=0.002, mu_scale=1e-4, offset_reduce="max"),
}


@pytest.mark.parametrize("name", list(MAXO))
def test_max_over_offsets_parity(name):
    cfg = MAXO[name]
    prob = _run(cfg)
    assert prob.flags() == _expected_flags(cfg)
    kept = {unit: check_unit(prob, unit, form="direct") for unit in range(cfg.n_units)}
    _check_oracle_compaction(prob, kept)


def test_max_over_offsets_full_size_sampled():
    """The Qwen3-8B-shaped workload with the maximum over its 17 offsets, in the
    benchmark's launch configuration (no per-query-head scores)."""
    cfg = C["qwen3_8b"].replace(name="qwen3_8b_max", offset_reduce="max")
    prob = _run(cfg, keep_raw=False)
    assert prob.flags() == 0
    kept = {}
    for unit, heads in ((0, [0, 5]), (cfg.n_units - 1, [3]), (17, [7])):
        log(f"[parity] {cfg.name}: checking unit {unit}")
        kept[unit] = check_unit(prob, unit, heads=heads, form="direct")
    _check_oracle_compaction(prob, kept)


@pytest.fixture(params=[L.SELECT_TILED, L.SELECT_PER_GROUP], ids=["tiled", "per_group"])
def strategy(request):
    prev = L.tria_select_strategy(request.param)
    yield request.param
    L.tria_select_strategy(prev)


@pytest.mark.parametrize("name", list(SMALL))
def test_select_strategies_agree(name):
    """The per-group and tiled selections keep bit-identical slots (the small cases
    have too few groups for the automatic choice to take the per-group kernel)."""
    cfg = SMALL[name]
    prev = L.tria_select_strategy(L.SELECT_TILED)
    try:
        prob = _run(cfg)
        ref_idx, ref_cnt = prob.idx.clone(), prob.cnt.clone()
        L.tria_select_strategy(L.SELECT_PER_GROUP)
        prob.idx.fill_(-7)
        prob.cnt.fill_(-7)
        prob.select()
        torch.cuda.synchronize()
        assert prob.flags() == _expected_flags(cfg)
        assert torch.equal(prob.cnt, ref_cnt)
        assert torch.equal(prob.idx, ref_idx)
    finally:
        L.tria_select_strategy(prev)


@pytest.mark.parametrize("name", ["q8_small", "lc_small", "bd_small"])
def test_small_raw_against_direct_form(name):
    """The literal 17-offset average, not only the folded oracle."""
    cfg = SMALL[name]
    prob = _run(cfg)
    unit = cfg.n_units - 1
    g = cfg.n_kv_heads - 1
    o_raw, _, _ = oracle_head(cfg, unit, g, form="direct")
    n = int(synth.units(cfg).lengths[unit])
    check_raw(prob.raw[unit, g * cfg.group:(g + 1) * cfg.group, :n].cpu().numpy(), o_raw, f"{name} direct")


def test_zero_statistics_break_ties_by_slot(strategy):
    """All-zero statistics give every key the score 0: the kept candidates must be
    the lowest slots (ties go to the lower slot)."""
    cfg = C["tiny"].replace(name="zero_stats", n_kv=3000, budget=900, sink=5, window=100, agg="max")
    prob = DeviceProblem(cfg)
    for t in (prob.q_re, prob.q_im, prob.q_abs):
        t.zero_()
    prob.run()
    torch.cuda.synchronize()
    F = cfg.head_dim // 2
    zero = np.zeros((cfg.n_layers, cfg.n_q_heads, F))
    kept = {0: check_unit(prob, 0, mu=zero.astype(complex), absm=zero)}
    for g in range(cfg.n_kv_heads):
        want = np.concatenate([np.arange(5), np.arange(5, 5 + 900 - 105), np.arange(2900, 3000)])
        np.testing.assert_array_equal(prob.kept(0, g), want)
    _check_oracle_compaction(prob, kept)


def test_duplicate_rows_tie_rule(strategy):
    """Keys that repeat every 97 slots score identically (a cached row's score
    depends on the row only), so the aggregates hold many exact ties around the
    threshold: every slot above the kept set's smallest candidate aggregate T is
    kept, none below it, and the tied slots kept are the lowest ones.  Checked on
    the GPU's own aggregates, and the strategies must agree bit for bit."""
    cfg = C["qwen3_8b"].replace(name="dup_rows", n_layers=1, n_kv_heads=2, n_kv=4000, budget=1000)
    prob = DeviceProblem(cfg)
    assert prob.paging is None
    idx = torch.arange(prob.K.shape[2], device=prob.K.device) % 97
    prob.K.copy_(prob.K[:, :, idx])
    prob.run()
    torch.cuda.synchronize()
    assert prob.flags() == 0
    n, B = int(synth.units(cfg).lengths[0]), int(synth.units(cfg).budget[0])
    prot = o.protected_mask(n, cfg.sink, cfg.window)
    for g in range(cfg.n_kv_heads):
        agg = prob.agg[0, g, :n].cpu().numpy()
        kept = prob.kept(0, g)
        assert kept.size == min(B, n)
        mask = np.zeros(n, bool)
        mask[kept] = True
        assert mask[prot].all()
        T = agg[mask & ~prot].min()
        assert mask[agg > T].all() and not mask[agg < T].any()
        tied = np.nonzero(agg == T)[0]
        n_tied_kept = int(mask[tied].sum())
        assert 1 <= n_tied_kept < tied.size, "the case should split a tie"
        np.testing.assert_array_equal(np.nonzero(mask[tied])[0], np.arange(n_tied_kept))
    ref_idx, ref_cnt = prob.idx.clone(), prob.cnt.clone()
    prev = L.tria_select_strategy(L.SELECT_PER_GROUP if strategy != L.SELECT_PER_GROUP else L.SELECT_TILED)
    try:
        prob.select()
        torch.cuda.synchronize()
        assert torch.equal(prob.idx, ref_idx) and torch.equal(prob.cnt, ref_cnt)
    finally:
        L.tria_select_strategy(prev)


def test_empty_and_zero_budget_units(strategy):
    cfg = C["batched_decode"].replace(name="empty", n_seqs=4, n_kv=700, ragged_min=100, window=0, sink=0)
    prob = DeviceProblem(cfg)
    prob.len[1] = 0
    prob.budget[2] = 0
    prob.run()
    torch.cuda.synchronize()
    assert prob.flags() == 0
    cnt = prob.cnt.cpu().numpy()
    assert cnt[1] == 0 and cnt[2] == 0
    assert (prob.idx[1].cpu().numpy() == -1).all() and (prob.idx[2].cpu().numpy() == -1).all()
    for unit in (0, 3):
        check_unit(prob, unit)


def test_many_units_with_empty_ones():
    """More units than the score kernel lists (520 > 512): every tile is claimed, also
    the empty ones past a unit's length.  Units of length 0 have no tile that would
    publish their moments; their tiles must finish without waiting (no expired wait,
    so no TRIA_FLAG_SYNC) and leave the other units' results as the oracle's."""
    cfg = C["batched_decode"].replace(name="many_units", n_seqs=520, n_kv=300, ragged_min=100, window=16)
    log(f"[parity] {cfg.name}: {cfg.n_units} units, every 37th emptied")
    prob = DeviceProblem(cfg)
    empty = list(range(5, cfg.n_units, 37))
    for unit in empty:
        prob.len[unit] = 0
    prob.run()
    torch.cuda.synchronize()
    prob.check_guards()
    assert prob.flags() == 0
    cnt = prob.cnt.cpu().numpy()
    assert all(cnt[unit] == 0 for unit in empty)
    kept = {}
    for unit in (0, 4, 6, 41, 43, 519):
        assert unit not in empty
        kept[unit] = check_unit(prob, unit)
    _check_oracle_compaction(prob, kept)


def test_device_flags_record_bad_metadata(strategy):
    """Out-of-contract device metadata is clamped by the kernels and reported."""
    cfg = C["batched_decode"].replace(name="flags", n_seqs=3, n_kv=500, ragged_min=200)
    prob = DeviceProblem(cfg)
    prob.len[0] = prob.n_max + 7        # clamped to n_max
    prob.unit_layer[1] = 5              # no such layer: coefficients are zero
    prob.budget[2] = 3                  # below sink + window while len > budget
    prob.run()
    torch.cuda.synchronize()
    f = prob.flags()
    assert f & L.FLAG_LEN and f & L.FLAG_LAYER and f & L.FLAG_BUDGET
    assert prob.flags() == 0            # reading clears the word
    assert int(prob.cnt[2].item()) == 3


def test_statistics_follow_the_unit_layer_map():
    """Each unit takes its statistics through its entry of the unit -> layer map, not
    through its own index.  Relabelling the layers (moving the statistics' layer axis
    and the map by the same permutation) leaves every output bit-identical; pointing
    several units at one layer scores each of them with that layer's statistics."""
    cfg = C["qwen3_8b"].replace(name="layer_map", n_layers=4, n_kv=3001, budget=700)
    log(f"[parity] layer map: {cfg.n_units} units")
    prob = DeviceProblem(cfg)
    names = ("agg", "idx", "cnt", "K", "V", "pos")

    def run():
        for t in (prob.agg, prob.idx, prob.cnt, prob.pos_out):
            t.fill_(-7)
        prob.K_out.view(torch.int16).fill_(-7)
        prob.V_out.view(torch.int16).fill_(-7)
        prob.run()
        torch.cuda.synchronize()
        assert prob.flags() == 0
        return [t.clone() for t in (prob.agg, prob.idx, prob.cnt, prob.K_out.view(torch.int16),
                                    prob.V_out.view(torch.int16), prob.pos_out)]

    ref = run()
    perm = np.array([2, 0, 3, 1])                    # old layer l gets label perm[l]
    pt = torch.from_numpy(perm).to(prob.dev)
    for t in (prob.q_re, prob.q_im, prob.q_abs):
        moved = torch.empty_like(t)
        moved[pt] = t
        t.copy_(moved)
    prob.unit_layer.copy_(pt[prob.unit_layer.long()].to(torch.int32))
    for r, g, what in zip(ref, run(), names):
        assert torch.equal(r, g), f"relabelled layers: {what} differs"

    # units 0, 1 and 3 on one layer, unit 2 on another (labels of the relabelled axis)
    shared = np.array([1, 1, 3, 1], np.int32)
    prob.unit_layer.copy_(torch.from_numpy(shared).to(prob.dev))
    run()
    re, im, ab = synth.q_stats(cfg)
    src = np.argsort(perm)[shared]                   # the original layer each unit now reads
    mu = (re.astype(np.float64) + 1j * im.astype(np.float64))[src]
    for unit in range(cfg.n_units):
        check_unit(prob, unit, mu=mu, absm=ab.astype(np.float64)[src])


# ----------------------------------------------------------------------------- full sizes

# pairs that are also checked with the literal offset loop (the direct form) and
# compacted on the host from regenerated rows
FULL_SAMPLES = {
    "qwen3_8b": [(0, 0), (17, 3), (35, 7)],
    "qwen3_32b": [(0, 0), (63, 7)],
    "batched_decode": [(0, 0), (37, 5), (63, 7)],
    "long_context": [(0, 5)],
}


def _nonconc_pair(cfg):
    nc = synth.nonconcentrated(cfg)
    rows = np.argwhere(nc)
    return (int(rows[0][0]), int(rows[0][1])) if rows.size else (0, 0)


@pytest.mark.parametrize("name,keep_raw", [(n, False) for n in FULL_SAMPLES] + [("qwen3_8b", True)])
def test_full_size_every_unit(name, keep_raw):
    """Every (unit, KV head) of the full-size workloads against the folded fp64 oracle
    (aggregates element by element, kept sets, and with keep_raw the per-query-head
    scores), in the benchmark's launch configuration when keep_raw is False; the
    oracle runs in a process pool over the host cores.  Compaction: every pair
    against a device gather of its source rows, sampled pairs on the host from
    regenerated rows and with the oracle's kept slots.  Sampled pairs are also
    scored with the literal loop over the offsets."""
    cfg = C[name]
    prob = _run(cfg, keep_raw=keep_raw)
    assert prob.flags() == 0
    u = synth.units(cfg)
    cnt = prob.cnt.cpu().numpy()
    np.testing.assert_array_equal(cnt, np.minimum(u.budget, u.lengths))
    agg = prob.agg.cpu().numpy()
    idx = prob.idx.cpu().numpy()
    raw = prob.raw.cpu().numpy() if keep_raw else None
    G = cfg.group
    pairs = [(unit, g) for unit in range(cfg.n_units) for g in range(cfg.n_kv_heads)]
    log(f"[parity] {name}: oracle over {len(pairs)} (unit, KV head) pairs")
    done = 0
    for (unit, g), o_raw, o_agg, o_kept in oracle_pairs(cfg, pairs, want_raw=keep_raw):
        n, k = int(u.lengths[unit]), int(cnt[unit])
        what = f"{name} unit {unit} kv {g}"
        if keep_raw:
            check_raw(raw[unit, g * G:(g + 1) * G, :n], o_raw, what)
        check_agg(agg[unit, g, :n], o_agg, what)
        check_kept(idx[unit, g, :k].astype(np.int64), o_kept, o_agg, n, int(u.budget[unit]), cfg.sink,
                   cfg.window, what)
        assert (idx[unit, g, k:] == -1).all(), what
        done += 1
        if done % 64 == 0:
            log(f"[parity] {name}: {done} pairs checked")
    assert done == len(pairs)
    check_compaction_on_device(prob, name)
    samples = list(FULL_SAMPLES[name])
    if name == "qwen3_32b":
        samples.append(_nonconc_pair(cfg))
    log(f"[parity] {name}: {len(samples)} pairs with the direct form")
    kept = {}
    for (unit, g), o_raw, o_agg, o_kept in oracle_pairs(cfg, samples, form="direct", want_raw=keep_raw):
        n, k = int(u.lengths[unit]), int(cnt[unit])
        what = f"{name} unit {unit} kv {g} (direct form)"
        if keep_raw:
            check_raw(raw[unit, g * G:(g + 1) * G, :n], o_raw, what)
        check_agg(agg[unit, g, :n], o_agg, what)
        g_kept = idx[unit, g, :k].astype(np.int64)
        check_kept(g_kept, o_kept, o_agg, n, int(u.budget[unit]), cfg.sink, cfg.window, what)
        check_compaction(prob, unit, g, g_kept, what)
        kept.setdefault(unit, {})[g] = o_kept
    _check_oracle_compaction(prob, kept)


def test_row_at_resident_capacity():
    """The longest row the score kernel takes: every tile of a (unit, KV head) must be
    resident at once, 512 workgroups of 2048-key tiles on MI355X, so one row of
    1,048,000 keys (512 tiles, the last one partial) against the oracle, with 100,000
    kept and compacted."""
    cfg = C["qwen3_8b"].replace(name="resident_max", n_layers=1, n_kv_heads=1, n_kv=1_048_000, budget=100_000)
    log(f"[parity] {cfg.name}: one row of {cfg.n_kv} keys")
    prob = _run(cfg)
    assert prob.flags() == 0
    kept = {0: check_unit(prob, 0)}
    _check_oracle_compaction(prob, kept)


# ----------------------------------------------------------------------------- schedule

SCHED = {
    "sched_dense": C["qwen3_8b"].replace(name="sched_dense", n_layers=4),
    "sched_g8": C["qwen3_32b"].replace(name="sched_g8", n_layers=2, n_kv=20000, budget=3000),
    "sched_paged": C["batched_decode"].replace(name="sched_paged", n_seqs=8),
}


def _tiles_per_row(prob, capfd):
    """Score tiles per (unit, KV head) that tria_score chose, read from its log line."""
    prev = L.tria_log(1)
    try:
        capfd.readouterr()
        prob.score()
        torch.cuda.synchronize()
        err = capfd.readouterr().err
    finally:
        L.tria_log(prev)
    m = re.search(r"tiles of \d+ keys \((\d+) per \(unit, KV head\)", err)
    assert m, err
    return int(m.group(1))


@pytest.mark.parametrize("name", list(SCHED))
def test_score_schedule_independence(name, capfd):
    """The score kernel's results do not depend on its persistent grid.  With the grid
    capped at the tiles of one (unit, KV head), each workgroup claims many tiles, often
    several of one (unit, KV head), and waits on far fewer peers than with the default
    grid (for G = 8 at this size: the single-buffer mode in several rounds).
    Aggregates, kept slots and compacted rows must be bit-identical."""
    cfg = SCHED[name]
    prob = _run(cfg)
    assert prob.flags() == 0
    n_tiles = _tiles_per_row(prob, capfd)
    ref = [t.clone() for t in (prob.agg, prob.idx, prob.cnt, prob.K_out, prob.V_out, prob.pos_out)]
    prev = L.tria_score_max_workgroups(0)
    try:
        for cap in (n_tiles, n_tiles + 3, 4 * n_tiles + 1):
            L.tria_score_max_workgroups(cap)
            for t in (prob.agg, prob.idx, prob.cnt, prob.K_out, prob.V_out, prob.pos_out):
                t.zero_()
            prob.run()
            torch.cuda.synchronize()
            assert prob.flags() == 0, cap
            u = synth.units(cfg)
            for unit in range(cfg.n_units):
                n = int(u.lengths[unit])
                assert torch.equal(prob.agg[unit, :, :n], ref[0][unit, :, :n]), (cap, unit)
            for got, want in zip((prob.idx, prob.cnt, prob.K_out, prob.V_out, prob.pos_out), ref[1:]):
                assert torch.equal(got, want), cap
        # a cap below one (unit, KV head)'s tiles is rejected before any launch
        L.tria_score_max_workgroups(n_tiles - 1)
        with pytest.raises(L.TriaError) as err:
            prob.score()
        assert err.value.status == L.TRIA_ESHAPE
    finally:
        L.tria_score_max_workgroups(prev)


def test_compaction_layout_paths_agree():
    """K and V through one block table take the batched compaction kernel; V through
    its own copy of the table takes the row-at-a-time kernel.  Both must copy the
    same bits."""
    cfg = C["batched_decode"].replace(name="compact_paths", n_seqs=3, n_kv=5000, ragged_min=1000)
    prob = _run(cfg)
    ref = [t.clone() for t in (prob.K_out, prob.V_out, prob.pos_out)]
    for t in (prob.K_out, prob.V_out, prob.pos_out):
        t.zero_()
    d, hkv, bs = cfg.head_dim, cfg.n_kv_heads, cfg.block_size
    bt2, dbt2 = prob.bt.clone(), prob.dbt.clone()
    v_view = L.make_view(prob.V, 0, d, hkv * d, bt2, bs, bt2.shape[1], prob.paging.n_blocks)
    vd_view = L.make_view(prob.V_out, 0, d, hkv * d, dbt2, bs, dbt2.shape[1], prob.paging.n_dst_blocks)
    L.tria_compact(prob.params, prob.k_view, v_view, prob.pos, 1, cfg.n_units, prob.n_max, prob.b_max, prob.len,
                   prob.idx, prob.cnt, prob.kd_view, vd_view, prob.pos_out, None)
    torch.cuda.synchronize()
    for got, want in zip((prob.K_out, prob.V_out, prob.pos_out), ref):
        assert torch.equal(got, want)


# ----------------------------------------------------------------------------- direct moments

DIRECT = ["q8_small", "q32_small", "bd_small", "lc_small", "d256_neox", "d64_inter", "g7", "short_units",
          "concentrated"]
DIRECT_MAX = ["q8_max", "bd_max", "lc_max", "concentrated_max"]


@pytest.mark.parametrize("name", DIRECT + DIRECT_MAX)
def test_moments_computed_directly(name):
    """With the moment exchange switched off (tria_score_wait_polls(-1)) every
    finalisation computes its group's moments straight from the K cache: the path a
    workgroup takes when its bounded wait runs out, so that results never depend on
    the tiles' workgroups being resident together.  Checked against the oracle like
    the small cases; TRIA_FLAG_SYNC records that the path ran."""
    cfg = SMALL[name] if name in SMALL else MAXO[name]
    prev = L.tria_score_wait_polls(-1)
    try:
        prob = _run(cfg)
        flags = prob.flags()
    finally:
        L.tria_score_wait_polls(prev)
    assert flags & L.FLAG_SYNC
    assert flags & ~L.FLAG_SYNC == _expected_flags(cfg)
    form = "direct" if cfg.offset_reduce == "max" else "folded"
    kept = {unit: check_unit(prob, unit, form=form) for unit in range(cfg.n_units)}
    _check_oracle_compaction(prob, kept)


def test_direct_moments_schedule_independent():
    """The direct path's moments run in a fixed order: aggregates, kept slots and
    compacted rows are bit-identical for every cap on the persistent grid."""
    cfg = SCHED["sched_g8"]
    prev = L.tria_score_wait_polls(-1)
    prev_cap = L.tria_score_max_workgroups(0)
    try:
        prob = _run(cfg)
        ref = [t.clone() for t in (prob.agg, prob.idx, prob.cnt, prob.K_out, prob.V_out, prob.pos_out)]
        n_tiles = -(-prob.n_max // 1024)
        L.tria_score_max_workgroups(n_tiles)
        for t in (prob.agg, prob.idx, prob.cnt, prob.K_out, prob.V_out, prob.pos_out):
            t.zero_()
        prob.run()
        torch.cuda.synchronize()
        assert prob.flags() & ~L.FLAG_SYNC == 0
        u = synth.units(cfg)
        for unit in range(cfg.n_units):
            n = int(u.lengths[unit])
            assert torch.equal(prob.agg[unit, :, :n], ref[0][unit, :, :n]), unit
        for got, want in zip((prob.idx, prob.cnt, prob.K_out, prob.V_out, prob.pos_out), ref[1:]):
            assert torch.equal(got, want)
        check_unit(prob, 1)
    finally:
        L.tria_score_wait_polls(prev)
        L.tria_score_max_workgroups(prev_cap)
