"""TRIA statistics files over the C ABI: save the calibrated query statistics, load
them back with an optional per-band mask folded in, and turn the per-layer budget
scales into per-unit budgets [Calib issue: stats files with magic 0x54524941,
versions 1..3, layer budget scales defaulting to 1.0; Fold note, sec. 7: a per-band
mask multiplies ||mu'_f||].  All the parsing, encoding and scaling is the library's
host code (tria_stats_*); this module reads and writes the bytes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import _lib as L


@dataclass
class Stats:
    version: int
    n_kv_heads: int
    q_mean_re: np.ndarray            # float32 [n_layers][n_heads][fc]
    q_mean_im: np.ndarray
    q_abs_mean: np.ndarray
    mrl: np.ndarray                  # zeros for a version-1 file
    layer_budget_scales: np.ndarray  # float32 [n_layers], 1.0 where the file has none

    @property
    def shape(self):
        return self.q_mean_re.shape

    def unit_budgets(self, unit_layer, budget: int) -> np.ndarray:
        """int32 per-unit budgets: round(budget * scale of the unit's layer)."""
        return L.tria_stats_layer_budgets(unit_layer, self.layer_budget_scales, budget)


def save(path: str, n_kv_heads: int, q_mean_re, q_mean_im, q_abs_mean, mrl=None, layer_budget_scales=None,
         version: int | None = None) -> int:
    """Writes a stats file (version 3 when scales are given, else 2 unless stated);
    returns its size in bytes."""
    if version is None:
        version = 3 if layer_budget_scales is not None else 2
    data = L.tria_stats_encode(version, n_kv_heads, q_mean_re, q_mean_im, q_abs_mean, mrl, layer_budget_scales)
    with open(path, "wb") as f:
        f.write(data)
    return len(data)


def load(path: str, band_mask=None) -> Stats:
    """Reads a stats file; with ``band_mask`` ([fc], >= 0) the mask is folded into the
    centres (the norm weights are unchanged)."""
    with open(path, "rb") as f:
        data = f.read()
    info, re, im, ab, mrl, scales = L.tria_stats_parse(data)
    if band_mask is not None:
        L.tria_stats_band_mask(band_mask, re, im, ab)
    return Stats(int(info.version), int(info.n_kv_heads), re, im, ab, mrl, scales)
