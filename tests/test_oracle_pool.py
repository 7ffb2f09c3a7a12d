"""The process pool the full-size GPU parity uses gives the oracle's own results."""
import numpy as np

from _parity import oracle_head, oracle_pairs
from key_importance_scoring_amd import synth


def test_pool_matches_serial_oracle():
    cfg = synth.CONFIGS["tiny"].replace(name="pool", n_kv=700, budget=300, window=64)
    pairs = [(0, 1), (0, 0)]
    got = list(oracle_pairs(cfg, pairs, want_raw=True, workers=2))
    assert [p for p, *_ in got] == pairs
    for (unit, g), raw, agg, kept in got:
        r, a, k = oracle_head(cfg, unit, g)
        np.testing.assert_array_equal(raw, r)
        np.testing.assert_array_equal(agg, a)
        np.testing.assert_array_equal(kept, k)
