"""tria_pass_noalloc, the pass on the library's own device array (for callers that
cannot allocate), against the three calls with a caller's workspace: two calls in a
row on one device, the second on a smaller input (paged), each compared element by
element with tria_score -> tria_select -> tria_compact on the same inputs, and the
first unit of each against the fp64 oracle."""
import numpy as np
import pytest
import torch

from _parity import check_unit, log
from key_importance_scoring_amd import _lib as L
from key_importance_scoring_amd import synth
from key_importance_scoring_amd.device import Guarded

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _noalloc(prob):
    """Runs tria_pass_noalloc on prob's inputs into outputs of its own (guarded)."""
    from key_importance_scoring_amd.device import DeviceProblem  # noqa: F401
    cfg = prob.cfg
    g = Guarded(prob.dev)
    agg = g.zeros(tuple(prob.agg.shape), torch.float32)
    idx = g.zeros(tuple(prob.idx.shape), torch.int32)
    cnt = g.zeros(tuple(prob.cnt.shape), torch.int32)
    k_out = g.zeros(tuple(prob.K_out.shape), torch.bfloat16)
    v_out = g.zeros(tuple(prob.V_out.shape), torch.bfloat16)
    pos_out = g.zeros(tuple(prob.pos_out.shape), torch.int32)
    flags = g.zeros((1,), torch.int32)
    d, hkv = cfg.head_dim, cfg.n_kv_heads
    if cfg.paged:
        bs, mdb = cfg.block_size, prob.dbt.shape[1]
        kd = L.make_view(k_out, 0, d, hkv * d, prob.dbt, bs, mdb, prob.paging.n_dst_blocks)
        vd = L.make_view(v_out, 0, d, hkv * d, prob.dbt, bs, mdb, prob.paging.n_dst_blocks)
    else:
        kd = L.make_view(k_out, hkv * prob.b_max * d, prob.b_max * d, d)
        vd = L.make_view(v_out, hkv * prob.b_max * d, prob.b_max * d, d)
    L.tria_pass_noalloc(prob.params, prob.k_view, prob.v_view, cfg.n_units, prob.n_max, prob.b_max, prob.len,
                        prob.unit_layer, prob.q_pos, prob.budget, prob.q_re, prob.q_im, prob.q_abs, prob.pos, 1, agg,
                        idx, cnt, kd, vd, pos_out, flags)
    torch.cuda.synchronize()
    g.check()
    return agg, idx, cnt, k_out, v_out, pos_out, int(flags[0].item())


def test_noalloc_matches_the_three_calls():
    from key_importance_scoring_amd.device import DeviceProblem
    cases = (C["qwen3_8b"].replace(name="noalloc_dense", n_layers=3, n_kv=9000, budget=1500),
             C["batched_decode"].replace(name="noalloc_paged", n_seqs=4, n_kv=3000, ragged_min=500))
    for cfg in cases:
        log(f"[noalloc] {cfg.name}: units={cfg.n_units} n_kv={cfg.n_kv} paged={cfg.paged}")
        prob = DeviceProblem(cfg, keep_raw=False)
        prob.run()
        torch.cuda.synchronize()
        assert prob.flags() == 0
        prob.check_guards()
        agg, idx, cnt, k_out, v_out, pos_out, flags = _noalloc(prob)
        assert flags == 0
        u = synth.units(cfg)
        for unit in range(cfg.n_units):
            n = int(u.lengths[unit])
            assert torch.equal(agg[unit, :, :n], prob.agg[unit, :, :n]), unit
        for got, want in ((idx, prob.idx), (cnt, prob.cnt), (k_out, prob.K_out), (v_out, prob.V_out),
                          (pos_out, prob.pos_out)):
            assert torch.equal(got, want)
        check_unit(prob, 0)
