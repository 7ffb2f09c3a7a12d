"""GPU parity of the calibration reduction (tria_calibrate) against the fp64 oracle.

Every (layer, query head, band) of the small cases is compared with
``oracle.calibrate`` on the same synthetic pre-RoPE query rows; the cases span
both pairings, head dims 64/128/256, one row, a whole 256-row chunk and ragged
tails.  The full-size case (a Qwen3-8B shaped stream of 8192 tokens, the
benchmark's workload) is checked on sampled heads.

Tolerance, derived from the arithmetic: a chunk's sums run in fp32 over at most
80 additions per value (d/16 lanes share a row; a lane adds 16-64 rows, then the
64-16 row partials are added) and then in fp64 over chunks, so each mean carries an
absolute error below 80 * 2^-24 ~ 5e-6 times the mean magnitude of its terms;
|q_f| and q_f / |q_f| (one 1-ulp reciprocal square root) add a few fp32 ulps.  The
means are therefore held to 1e-5 * E|q_f| (|Re q_f|, |Im q_f| <= |q_f|), the
unit-phasor mean (terms of magnitude <= 1) to 1e-5 absolute, and the ratio r to
2e-5 absolute (an error in |E q_f| and in E|q_f| of 1e-5 * E|q_f| each).
"""
import numpy as np
import pytest
import torch

from _parity import log
from oracle import tria_oracle as o
from key_importance_scoring_amd import synth
from key_importance_scoring_amd.device import calibrate, params_for

pytestmark = pytest.mark.gpu

C = synth.CONFIGS
CASES = {
    "tiny_T1000": (C["tiny"], 1000),
    "q8_T777": (C["qwen3_8b"].replace(name="q8_cal", n_layers=2), 777),
    "lc_inter_T300": (C["long_context"].replace(name="lc_cal", n_kv_heads=2), 300),
    "d256_neox_T257": (C["qwen3_8b"].replace(name="d256n_cal", head_dim=256, n_layers=1, n_kv_heads=2), 257),
    "d256_inter_T256": (C["long_context"].replace(name="d256i_cal", head_dim=256, n_kv_heads=1, group=3), 256),
    "d64_inter_T1": (C["tiny"].replace(name="d64i_cal", pairing="interleaved"), 1),
    "d64_inter_T513": (C["tiny"].replace(name="d64i_cal2", pairing="interleaved", n_layers=2), 513),
}
FULL = C["qwen3_8b"]
FULL_T = 8192


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _upload(q_bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).to("cuda:0")


def _check_head(got: dict, l: int, h: int, rows: np.ndarray, pairing: str, r: bool = True, mrl: bool = True):
    mr, mi, ab, rr, ml = o.calibrate(rows, pairing)
    g = {k: (v[l, h].double().cpu().numpy() if v is not None else None) for k, v in got.items()}
    tol = 1e-5 * ab + 1e-30
    for name, want in (("q_mean_re", mr), ("q_mean_im", mi), ("q_abs_mean", ab)):
        err = np.abs(g[name] - want)
        assert np.all(err <= tol), (name, l, h, float(err.max()), int(np.argmax(err - tol)))
    if r:
        assert np.all(np.abs(g["r"] - rr) <= 2e-5), ("r", l, h, float(np.abs(g["r"] - rr).max()))
    if mrl:
        assert np.all(np.abs(g["mrl"] - ml) <= 1e-5), ("mrl", l, h, float(np.abs(g["mrl"] - ml).max()))


@pytest.mark.parametrize("name", list(CASES))
def test_calibration_matches_oracle(name):
    cfg, T = CASES[name]
    log(f"[calib] {name}: L={cfg.n_layers} Hq={cfg.n_q_heads} d={cfg.head_dim} T={T} pairing={cfg.pairing}")
    q = synth.query_stream(cfg, T, workers=1)
    got = calibrate(params_for(cfg), _upload(q))
    torch.cuda.synchronize()
    for l in range(cfg.n_layers):
        for h in range(cfg.n_q_heads):
            _check_head(got, l, h, q[l, h], cfg.pairing)


def test_strided_layout_is_bit_identical():
    """A token-major [T][L][Hq][d] buffer viewed as [L][Hq][T][d] gives the same bits
    as the contiguous stream: the summation order depends on the token index only."""
    cfg, T = CASES["q8_T777"]
    log(f"[calib] strided: T={T}")
    q = synth.query_stream(cfg, T, workers=1)
    p = params_for(cfg)
    a = calibrate(p, _upload(q))
    tm = _upload(np.ascontiguousarray(q.transpose(2, 0, 1, 3)))     # [T][L][Hq][d]
    b = calibrate(p, tm.permute(1, 2, 0, 3))
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_optional_outputs_may_be_null():
    cfg, T = CASES["tiny_T1000"]
    q = synth.query_stream(cfg, T, workers=1)
    p = params_for(cfg)
    full = calibrate(p, _upload(q))
    part = calibrate(p, _upload(q), want_r=False, want_mrl=False)
    torch.cuda.synchronize()
    assert part["r"] is None and part["mrl"] is None
    for k in ("q_mean_re", "q_mean_im", "q_abs_mean"):
        assert torch.equal(full[k], part[k]), k


def test_degenerate_streams():
    """Zero rows give zeros everywhere (r and mrl take 0 where |q_f| = 0); identical
    rows give r = mrl = 1 on every non-zero band and means equal to the row."""
    cfg = C["tiny"].replace(name="degenerate")
    T, d = 700, cfg.head_dim
    p = params_for(cfg)
    zeros = np.zeros((cfg.n_layers, cfg.n_q_heads, T, d), np.uint16)
    z = calibrate(p, _upload(zeros))
    torch.cuda.synchronize()
    for k, v in z.items():
        assert torch.count_nonzero(v).item() == 0, k

    rng = np.random.default_rng(7)
    row = synth.f32_to_bf16_bits(rng.standard_normal(d).astype(np.float32))
    row[[0, d // 2]] = 0                            # band 0 (NEOX pairing) is zero
    row[[1, 2]] = 0                                 # bands 1, 2: real part zero
    same = np.broadcast_to(row, (cfg.n_layers, cfg.n_q_heads, T, d)).copy()
    s = calibrate(p, _upload(same))
    torch.cuda.synchronize()
    for l in range(cfg.n_layers):
        for h in range(cfg.n_q_heads):
            _check_head(s, l, h, same[l, h], cfg.pairing)
    mr, mi, ab, rr, ml = o.calibrate(same[0, 0], cfg.pairing)
    nz = ab > 0
    assert not nz[0] and nz[1:].all()
    assert np.all(np.abs(s["r"][0, 0].cpu().numpy()[nz] - 1.0) <= 2e-5)
    assert np.all(np.abs(s["mrl"][0, 0].cpu().numpy()[nz] - 1.0) <= 1e-5)


def test_full_size_sampled_heads():
    """The benchmark's stream (Qwen3-8B: 36 layers x 32 query heads x 8192 tokens x
    d 128, NEOX), every head computed on the GPU; sampled heads against the oracle."""
    cfg, T = FULL, FULL_T
    log(f"[calib] full size: L={cfg.n_layers} Hq={cfg.n_q_heads} T={T}")
    q = synth.query_stream(cfg, T)
    got = calibrate(params_for(cfg), _upload(q))
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    heads = {(0, 0), (cfg.n_layers - 1, cfg.n_q_heads - 1)}
    heads |= {(int(rng.integers(cfg.n_layers)), int(rng.integers(cfg.n_q_heads))) for _ in range(6)}
    for l, h in sorted(heads):
        _check_head(got, l, h, q[l, h], cfg.pairing)
