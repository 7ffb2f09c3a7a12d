"""Comparison of the HIP pass against the fp64 oracle, unit by unit.

Tolerances (fp32 accumulation on the device, fp64 in the oracle):
* raw score of query head h, slot i:  |g - o| <= 1e-3 * max(|o|, rms_h(o))
* aggregate of a candidate slot:      |g - o| <= 1e-3 * max(|o|, 1); protected slots are +inf on both sides
* kept slots: the two sets have min(B, n) elements, the GPU's are ascending and
  unique and hold every protected slot (when B >= protected), and any slot in
  only one of them has an oracle aggregate within 1e-3 * max(1, |T|) of the
  oracle's threshold T (the smallest kept candidate aggregate): such slots are
  ordered by rounding, not by the method
* compacted K, V rows and positions: bit-exact against the source rows at the
  GPU's own kept slots, and (through a second tria_compact call) at the oracle's.
"""
from __future__ import annotations

import functools
import sys

import numpy as np

from oracle import tria_oracle as o
from key_importance_scoring_amd import synth

RAW_TOL = 1e-3
AGG_TOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=8)
def _stats(cfg):
    re, im, ab = synth.q_stats(cfg)
    return re.astype(np.float64) + 1j * im.astype(np.float64), ab.astype(np.float64)


def oracle_head(cfg, unit: int, g: int, form: str = "folded", mu=None, absm=None):
    """Oracle raw [G][n], aggregate [n] and kept slots of one (unit, KV head)."""
    u = synth.units(cfg)
    n = int(u.lengths[unit])
    layer = int(u.unit_layer[unit])
    if mu is None:
        mu, absm = _stats(cfg)
    rows = o.bf16_bits_to_f64(synth.key_rows(cfg, unit, g))
    pos = synth.positions(cfg, unit)
    G = cfg.group
    raw = np.stack([o.score_head(rows, pos, int(u.q_pos[unit]), mu[layer, h], absm[layer, h], cfg.head_dim,
                                 cfg.pairing, cfg.rope_base, cfg.offsets, form, cfg.offset_reduce)
                    for h in range(g * G, (g + 1) * G)]) if n else np.zeros((G, 0))
    agg = o.aggregate_unit(raw, n, G, cfg.sink, cfg.window, cfg.agg)[0] if n else np.zeros(0)
    kept = o.select(agg, int(u.budget[unit])) if n else np.zeros(0, np.int64)
    return raw, agg, kept


def check_raw(g_raw: np.ndarray, o_raw: np.ndarray, what: str) -> None:
    for h in range(o_raw.shape[0]):
        ob = o_raw[h]
        if ob.size == 0:
            continue
        rms = float(np.sqrt(np.mean(ob ** 2)))
        tol = RAW_TOL * np.maximum(np.abs(ob), rms)
        err = np.abs(g_raw[h].astype(np.float64) - ob)
        bad = np.nonzero(err > tol)[0]
        assert bad.size == 0, (f"{what} raw head {h}: {bad.size} slots off, first {bad[:5]}, "
                               f"gpu {g_raw[h][bad[:5]]}, oracle {ob[bad[:5]]}")


def check_agg(g_agg: np.ndarray, o_agg: np.ndarray, what: str) -> None:
    inf_o = np.isinf(o_agg)
    assert np.array_equal(np.isinf(g_agg) & (g_agg > 0), inf_o), f"{what}: protected slots differ"
    c = ~inf_o
    err = np.abs(g_agg[c].astype(np.float64) - o_agg[c])
    tol = AGG_TOL * np.maximum(np.abs(o_agg[c]), 1.0)
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, f"{what} agg: {bad.size} slots off, max err {err.max()}"


def check_kept(g_kept: np.ndarray, o_kept: np.ndarray, o_agg: np.ndarray, n: int, budget: int, sink: int,
               window: int, what: str) -> None:
    want = min(budget, n)
    assert g_kept.size == want, f"{what}: kept {g_kept.size} != {want}"
    assert np.all(np.diff(g_kept) > 0), f"{what}: kept slots not ascending/unique"
    assert g_kept.size == 0 or (g_kept[0] >= 0 and g_kept[-1] < n), f"{what}: kept slot out of range"
    prot = np.nonzero(o.protected_mask(n, sink, window))[0]
    if budget >= prot.size:
        assert np.isin(prot, g_kept).all(), f"{what}: a protected slot was dropped"
    diff = np.setxor1d(g_kept, o_kept)
    if diff.size:
        T = o.kth_threshold(o_agg, n, budget, sink, window)
        near = np.abs(o_agg[diff] - T) <= AGG_TOL * max(1.0, abs(T))
        assert near.all(), (f"{what}: {int((~near).sum())} kept slots differ away from the threshold "
                            f"{T}: {diff[~near][:8]}")


def check_compaction(prob, unit: int, g: int, kept: np.ndarray, what: str) -> None:
    cfg = prob.cfg
    k_rows = synth.key_rows(cfg, unit, g)
    v_rows = synth.value_rows(cfg, unit, g)
    pos = synth.positions(cfg, unit)
    m = kept.size
    np.testing.assert_array_equal(prob.out_rows("k", unit, g, m), o.compact(k_rows, kept), err_msg=f"{what} K")
    np.testing.assert_array_equal(prob.out_rows("v", unit, g, m), o.compact(v_rows, kept), err_msg=f"{what} V")
    np.testing.assert_array_equal(prob.pos_out[unit, g, :m].cpu().numpy(), o.compact(pos, kept),
                                  err_msg=f"{what} pos")


def _pool_init():
    """Worker set-up: one BLAS thread per process (the pool already spans the cores)."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _oracle_pair(args):
    cfg, unit, g, form, want_raw = args
    raw, agg, kept = oracle_head(cfg, unit, g, form)
    return (raw if want_raw else None), agg, kept


def oracle_pairs(cfg, pairs, form: str = "folded", want_raw: bool = False, workers: int | None = None):
    """oracle_head for every (unit, KV head) in `pairs`, in a process pool over the
    host cores (spawned processes; at most 16).  Yields (pair, raw or None, agg,
    kept) in the order of `pairs`."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import os
    workers = workers or max(1, min(16, os.cpu_count() or 1))
    jobs = [(cfg, unit, g, form, want_raw) for unit, g in pairs]
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                                initializer=_pool_init) as ex:
        for pair, res in zip(pairs, ex.map(_oracle_pair, jobs, chunksize=2)):
            yield (pair, *res)


def check_compaction_on_device(prob, what: str) -> None:
    """Every (unit, KV head): the compacted K and V rows and positions equal the
    source's rows at the kept slots, gathered by torch on the device (an independent
    gather), for j < cnt[u]."""
    import torch
    cfg = prob.cfg
    d, bs = cfg.head_dim, cfg.block_size
    cnt = prob.cnt.cpu().numpy()
    for unit in range(cfg.n_units):
        k = int(cnt[unit])
        if k == 0:
            continue
        ix = prob.idx[unit, :, :k].long()                              # [Hkv][k]
        heads = torch.arange(cfg.n_kv_heads, device=ix.device)[:, None]
        j = torch.arange(k, device=ix.device)[None, :]
        for which in ("k", "v"):
            src = prob.K if which == "k" else prob.V
            dst = prob.K_out if which == "k" else prob.V_out
            if cfg.paged:
                bt, dbt = prob.bt[unit].long(), prob.dbt[unit].long()
                want = src[bt[ix // bs], ix % bs, heads]
                got = dst[dbt[j // bs], j % bs, heads]
            else:
                want = src[unit, heads, ix]
                got = dst[unit, :, :k]
            assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{what} unit {unit}: {which} rows"
        want_pos = prob.pos[unit, 0][ix]
        assert torch.equal(prob.pos_out[unit, :, :k], want_pos), f"{what} unit {unit}: positions"


def check_unit(prob, unit: int, heads=None, form: str = "folded", mu=None, absm=None):
    """Full comparison of one unit (optionally a subset of its KV heads).  Returns the
    oracle kept sets {kv_head: slots}."""
    cfg = prob.cfg
    u = synth.units(cfg)
    n = int(u.lengths[unit])
    B = int(u.budget[unit])
    G = cfg.group
    heads = range(cfg.n_kv_heads) if heads is None else heads
    assert int(prob.cnt[unit].item()) == min(B, n)
    kept_o = {}
    for g in heads:
        what = f"{cfg.name} unit {unit} kv {g}"
        o_raw, o_agg, o_kept = oracle_head(cfg, unit, g, form, mu, absm)
        if prob.raw is not None:
            check_raw(prob.raw[unit, g * G:(g + 1) * G, :n].cpu().numpy(), o_raw, what)
        check_agg(prob.agg[unit, g, :n].cpu().numpy(), o_agg, what)
        g_kept = prob.kept(unit, g)
        check_kept(g_kept, o_kept, o_agg, n, B, cfg.sink, cfg.window, what)
        check_compaction(prob, unit, g, g_kept, what)
        kept_o[g] = o_kept
    return kept_o
