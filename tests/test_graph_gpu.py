"""The pass under HIP graph capture: tria_score -> tria_select -> tria_compact make no
allocation, memset or synchronisation, so a caller can capture them once and replay
them.  Every replay, with the program's own eager work and synchronisations between
replays, must give bit-identical aggregates, kept slots, counts and compacted rows to
the eager calls (the maximum over offsets, a paged cache and the single-buffer score
kernel included).
"""
import pytest
import torch

from _parity import log
from key_importance_scoring_amd import _lib as L
from key_importance_scoring_amd import synth
from key_importance_scoring_amd.device import DeviceProblem

pytestmark = pytest.mark.gpu

C = synth.CONFIGS

CASES = {
    "q8_mean": C["qwen3_8b"].replace(name="graph_q8", n_layers=2, n_kv=5003, budget=1000),
    "bd_paged_max": C["batched_decode"].replace(name="graph_bd", n_seqs=5, n_kv=3000, ragged_min=500,
                                                offset_reduce="max"),
    # G = 8, dense: the single-buffer score kernel
    "lc_single": C["long_context"].replace(name="graph_lc", n_kv=6000, budget=600),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


def _outputs(prob):
    # K and V as bit patterns: rows the pass leaves untouched hold the scramble value,
    # a bf16 NaN, which a value comparison would never find equal to itself
    return [t.clone() for t in (prob.agg, prob.idx, prob.cnt, prob.K_out.view(torch.int16),
                                prob.V_out.view(torch.int16), prob.pos_out)]


def _scramble(prob):
    for t in (prob.agg, prob.idx, prob.cnt, prob.pos_out):
        t.fill_(-7)
    prob.K_out.view(torch.int16).fill_(-7)
    prob.V_out.view(torch.int16).fill_(-7)


@pytest.mark.parametrize("name", list(CASES))
def test_captured_pass_replays_match_eager(name):
    cfg = CASES[name]
    log(f"[graph] {name}: units={cfg.n_units} paged={cfg.paged} reduce={cfg.offset_reduce}")
    prob = DeviceProblem(cfg, keep_raw=False)
    _scramble(prob)        # regions the pass leaves untouched hold the same bytes in every run
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prob.run(side)                               # eager reference, on a side stream
    side.synchronize()
    assert prob.flags() == 0
    ref = _outputs(prob)

    graph = torch.cuda.CUDAGraph()
    _scramble(prob)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        prob.run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for replay in range(4):
        _scramble(prob)                              # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(prob)
        for r, g, what in zip(ref, got, ("agg", "idx", "cnt", "K", "V", "pos")):
            assert torch.equal(r, g), f"{name} replay {replay}: {what} differs"
    assert prob.flags() == 0
