"""fp64 CPU oracle for the TriAttention score -> select -> compact pass.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call this
module: only the tests, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP library and never reads a value
produced by it.

Everything is plain NumPy in float64, written for a reader to check by eye
against the pages; speed is not a goal.  Sources and how they are cited:

* [Fold note]  academ.us article 2607.13051, the short note that restates the
  TriAttention score and folds its future-offset average (sections 2-7,
  Eqs. 1-8).  The authority on what is computed.
* [Blog]  "TriAttention, or: what a rotating query already knows"
  (ghidav.me), sections "The Solution" and "The Method".
* [Calib issue]  GitHub issue "Request: publish TriAttention calibration script
  (TRIA v2/v3 stats.bin producer)" on domvox/llama.cpp-turboquant-hip: the
  band pairing conventions and the runtime log of the llama.cpp port.
* [Explainer]  repo-explainer.com article "TriAttention: The KV Cache
  Compressor That Reads Long Reasoning in the Frequency Domain" (inverting RoPE
  on cached keys).

Readings taken where the pages are silent (each one is also listed with its
reason in the design notes of the repository):

* S_norm = sum_f (E|q_f| - |E[q_f]|) |k_f|  (an assumption; the Blog says the
  norm term weighs a band in proportion to 1 - R_f with R_f = |E q_f| / E|q_f|,
  and the Fold note only says it does not depend on the distance).
* The current query sits at ``q_pos`` (the newest cached key); the future
  queries sit at ``q_pos + delta`` for delta in D.
* Protected slots: the first ``sink`` slots and the last ``window`` slots of
  the unit.  Candidates are all other slots.
* z-normalisation per q-head over the candidates, population std (ddof 0),
  z = (s - mean) / max(std, 1e-12); then GQA aggregation (mean or max) of the
  group's z onto the KV head (q-head h belongs to KV head h // G).
* Budget B counts every kept slot, protected ones included; kept count is
  min(B, n).  Protected slots rank above every candidate; among equal
  aggregates the lower slot wins.  Kept slots are reported in ascending order.
* Calibration: the concentration R_f is |E q_f| / E|q_f| (the ratio the norm
  term's weight E|q_f| (1 - R_f) needs); the pages name it a mean resultant
  length, whose circular-statistics form |E[q_f / |q_f|]| is returned beside it.

Parity pins (tests/test_oracle_pins.py) tie each function below to closed forms,
textbook routines, invariants or brute force.  No function here is left
unpinned.
"""
from __future__ import annotations

import numpy as np

NEOX = "neox"
INTERLEAVED = "interleaved"
SIGMA_FLOOR = 1e-12


# ----------------------------------------------------------------------------- inputs

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def band_frequencies(head_dim: int, theta: float) -> np.ndarray:
    """omega_f = theta^(-2f/d), f = 0 .. d/2-1.  [Fold note, sec. 2, Eq. 2 bullet list]"""
    f = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * f / head_dim)


def complex_bands(rows: np.ndarray, pairing: str) -> np.ndarray:
    """Real rows [..., d] -> complex bands [..., d/2].

    NEOX pairs dim f with dim f + d/2; the interleaved (NORM) pairing pairs dim
    2f with dim 2f+1.  [Calib issue, "RoPE complex pairing matches the model's
    rope_type"]
    """
    rows = np.asarray(rows, dtype=np.float64)
    d = rows.shape[-1]
    F = d // 2
    if pairing == NEOX:
        return rows[..., :F] + 1j * rows[..., F:]
    if pairing == INTERLEAVED:
        return rows[..., 0::2] + 1j * rows[..., 1::2]
    raise ValueError(f"unknown pairing {pairing!r}")


def invert_rope(k_rot: np.ndarray, pos: np.ndarray, omega: np.ndarray) -> np.ndarray:
    """Undo the rotary turn of cached keys: k_f = k_rot_f * e^{-i omega_f p_k}.

    The rotation is a multiplication by e^{i omega_f p} [Fold note, sec. 2.0.0.3
    fact 3]; its inverse is the conjugate turn.  The score is evaluated in the
    pre-rotation space [Fold note, sec. 2.0.0.1; Explainer, "inverts RoPE"].
    ``k_rot`` is [n][F], ``pos`` is [n].
    """
    pos = np.asarray(pos, dtype=np.float64)
    return k_rot * np.exp(-1j * np.outer(pos, omega))


# ----------------------------------------------------------------------------- score

def s_trig_direct(mu: np.ndarray, k: np.ndarray, dist: np.ndarray, offsets, omega: np.ndarray) -> np.ndarray:
    """Offset-averaged trigonometric term, computed literally.

    For each future offset delta in D, evaluate the band sum of Eq. 2 at
    distance Delta + delta,
        S_trig(k, Delta) = sum_f |E q_f| |k_f| cos(omega_f Delta + phi_f),
        phi_f = arg E[q_f] - arg k_f,
    and average over D (Eq. 4).  [Fold note, Eqs. 2 and 4]

    ``mu`` [F] complex query centre, ``k`` [n][F] pre-rotation key bands,
    ``dist`` [n] the distances Delta = q_pos - p_k.
    """
    mag = np.abs(mu)[None, :] * np.abs(k)                       # [n][F]
    phi = np.angle(mu)[None, :] - np.angle(k)                   # [n][F]
    total = np.zeros(k.shape[0], dtype=np.float64)
    offsets = list(offsets)
    for delta in offsets:
        ang = np.outer(np.asarray(dist, np.float64) + float(delta), omega) + phi
        total += np.sum(mag * np.cos(ang), axis=1)
    return total / len(offsets)


def s_trig_direct_max(mu: np.ndarray, k: np.ndarray, dist: np.ndarray, offsets, omega: np.ndarray) -> np.ndarray:
    """The variant that takes the maximum over the future offsets instead of the
    mean: max over delta in D of the band sum of Eq. 2 at distance Delta + delta.
    Not linear in the offsets, so no fold applies; evaluated literally, offset by
    offset.  [Fold note, sec. 4: the non-default maximum-over-offsets variant;
    Eq. 2 for each term]"""
    mag = np.abs(mu)[None, :] * np.abs(k)                       # [n][F]
    phi = np.angle(mu)[None, :] - np.angle(k)                   # [n][F]
    best = np.full(k.shape[0], -np.inf, dtype=np.float64)
    for delta in list(offsets):
        ang = np.outer(np.asarray(dist, np.float64) + float(delta), omega) + phi
        best = np.maximum(best, np.sum(mag * np.cos(ang), axis=1))
    return best


def s_trig_phasor(mu: np.ndarray, k: np.ndarray, dist: np.ndarray, offsets, omega: np.ndarray) -> np.ndarray:
    """Same quantity via the phasor form Re sum_f E[q_f] conj(k_f) e^{i omega_f Delta}
    (Eq. 3), averaged over D (Eq. 4).  [Fold note, Eqs. 3 and 4]"""
    total = np.zeros(k.shape[0], dtype=np.float64)
    offsets = list(offsets)
    for delta in offsets:
        rot = np.exp(1j * np.outer(np.asarray(dist, np.float64) + float(delta), omega))
        total += np.real(np.sum(mu[None, :] * np.conj(k) * rot, axis=1))
    return total / len(offsets)


def offset_weights(omega: np.ndarray, offsets) -> np.ndarray:
    """W_f = (1/|D|) sum_{delta in D} e^{i omega_f delta}.  [Fold note, Eq. 6]"""
    offsets = np.asarray(list(offsets), dtype=np.float64)
    return np.mean(np.exp(1j * np.outer(offsets, omega)), axis=0)


def s_trig_folded(mu: np.ndarray, k: np.ndarray, dist: np.ndarray, offsets, omega: np.ndarray) -> np.ndarray:
    """Folded form: one evaluation of Eq. 2 with the centre replaced by the
    offset-averaged centre mu'_f = E[q_f] W_f.  [Fold note, Eq. 7]"""
    mu_p = mu * offset_weights(omega, offsets)
    mag = np.abs(mu_p)[None, :] * np.abs(k)
    phi = np.angle(mu_p)[None, :] - np.angle(k)
    ang = np.outer(np.asarray(dist, np.float64), omega) + phi
    return np.sum(mag * np.cos(ang), axis=1)


def s_trig_realmap(mu: np.ndarray, k: np.ndarray, dist: np.ndarray, offsets, omega: np.ndarray) -> np.ndarray:
    """Real-coefficient form: a_f = |E q||k| cos phi, b_f = -|E q||k| sin phi,
    mapped by [[A, B], [-B, A]] with A = Re W_f, B = Im W_f, then
    sum_f a'_f cos(omega_f Delta) + b'_f sin(omega_f Delta).  [Fold note, sec. 7, Eq. 8]"""
    W = offset_weights(omega, offsets)
    A, B = W.real[None, :], W.imag[None, :]
    mag = np.abs(mu)[None, :] * np.abs(k)
    phi = np.angle(mu)[None, :] - np.angle(k)
    a = mag * np.cos(phi)
    b = -mag * np.sin(phi)
    a2 = A * a + B * b
    b2 = -B * a + A * b
    ang = np.outer(np.asarray(dist, np.float64), omega)
    return np.sum(a2 * np.cos(ang) + b2 * np.sin(ang), axis=1)


def s_norm(mu: np.ndarray, abs_mean: np.ndarray, k: np.ndarray) -> np.ndarray:
    """S_norm(k) = sum_f (E|q_f| - |E[q_f]|) |k_f|.

    Distance-independent [Fold note, sec. 2.0.0.2 after Eq. 2], weighting each
    band by E|q_f| (1 - R_f) [Blog, "The Method": the norm term contributes in
    proportion to 1 - R_f].  The exact form is the declared reading.
    """
    w = np.asarray(abs_mean, np.float64) - np.abs(mu)
    return np.abs(k) @ w


S_TRIG_FORMS = {
    "direct": s_trig_direct,
    "phasor": s_trig_phasor,
    "folded": s_trig_folded,
    "realmap": s_trig_realmap,
}


def score_head(rows: np.ndarray, pos: np.ndarray, q_pos: int, mu: np.ndarray, abs_mean: np.ndarray,
               head_dim: int, pairing: str, theta: float, offsets, form: str = "folded",
               reduce: str = "mean") -> np.ndarray:
    """S~(k) = (offset-averaged S_trig) + S_norm for every cached key of one KV head,
    seen by one q-head's calibrated centre.  [Fold note, Eqs. 1, 4, 6]

    ``rows`` [n][d] real post-rotation keys (fp64), ``pos`` [n] key positions,
    ``q_pos`` the current query position, ``mu`` [F] complex centre,
    ``abs_mean`` [F] the calibrated E|q_f|.  ``reduce="max"`` takes the maximum
    over the offsets instead (the direct form only; S_norm does not depend on the
    offset, so max_delta (S_trig + S_norm) = max_delta S_trig + S_norm).
    """
    omega = band_frequencies(head_dim, theta)
    k = invert_rope(complex_bands(rows, pairing), pos, omega)
    dist = float(q_pos) - np.asarray(pos, np.float64)
    if reduce == "max":
        trig = s_trig_direct_max(mu, k, dist, offsets, omega)
    elif reduce == "mean":
        trig = S_TRIG_FORMS[form](mu, k, dist, offsets, omega)
    else:
        raise ValueError(f"unknown offset reduction {reduce!r}")
    return trig + s_norm(mu, abs_mean, k)


# ----------------------------------------------------------------------------- selection

def protected_mask(n: int, sink: int, window: int) -> np.ndarray:
    """Slots always kept: the first ``sink`` slots (attention sinks) and the last
    ``window`` slots (the recent window).  The llama.cpp port scores only
    n_old = n_kv - window keys [Calib issue, runtime log]."""
    m = np.zeros(n, dtype=bool)
    m[:min(sink, n)] = True
    m[max(0, n - window):] = True
    return m


def znorm(scores: np.ndarray, candidates: np.ndarray) -> np.ndarray:
    """Per-q-head z-score over the candidate slots (population std, floored).
    [Calib issue: the port's scoring does GQA aggregation and z-norm]"""
    s = np.asarray(scores, np.float64)
    c = s[candidates]
    if c.size == 0:
        return np.zeros_like(s)
    m = np.mean(c)
    sd = np.sqrt(np.mean((c - m) ** 2))
    return (s - m) / max(sd, SIGMA_FLOOR)


def aggregate(z_group: np.ndarray, how: str) -> np.ndarray:
    """Grouped-query aggregation of the group's z-scores onto the KV head.
    [Fold note, sec. 4: normalize-then-max; mean is the other variant asked for]"""
    z_group = np.asarray(z_group, np.float64)
    if how == "max":
        return np.max(z_group, axis=0)
    if how == "mean":
        return np.mean(z_group, axis=0)
    raise ValueError(how)


def aggregate_unit(raw: np.ndarray, n: int, group: int, sink: int, window: int, how: str) -> np.ndarray:
    """raw [Hq][n] -> aggregate [Hkv][n]; protected slots get +inf."""
    Hq = raw.shape[0]
    prot = protected_mask(n, sink, window)
    cand = ~prot
    out = np.empty((Hq // group, n), np.float64)
    for g in range(Hq // group):
        z = np.stack([znorm(raw[h, :n], cand) for h in range(g * group, (g + 1) * group)])
        out[g] = aggregate(z, how)
        out[g, prot] = np.inf
    return out


def select(agg: np.ndarray, budget: int) -> np.ndarray:
    """Keep the top-B slots of one KV head ("Sort. Keep the top-B. Drop the rest."
    [Blog, "The Method"]).  A full sort by (aggregate descending, slot ascending);
    returns the kept slots in ascending order."""
    n = agg.shape[0]
    order = sorted(range(n), key=lambda i: (-agg[i], i))
    return np.array(sorted(order[:min(budget, n)]), dtype=np.int64)


def compact(rows: np.ndarray, kept: np.ndarray) -> np.ndarray:
    """Keep only the kept rows, in kept order (a plain gather; bit copy)."""
    return np.take(rows, kept, axis=0)


# ----------------------------------------------------------------------------- whole unit

def run_unit(k_bits: np.ndarray, pos: np.ndarray, q_pos: int, q_mean_re: np.ndarray, q_mean_im: np.ndarray,
             q_abs_mean: np.ndarray, *, head_dim: int, group: int, pairing: str, theta: float, offsets,
             sink: int, window: int, agg: str, budget: int, form: str = "folded", reduce: str = "mean"):
    """The whole pass for one unit (one layer of one sequence).

    ``k_bits`` [Hkv][n][d] bf16 bits of the cached keys, ``pos`` [n] or
    [Hkv][n] key positions, ``q_mean_*`` / ``q_abs_mean`` [Hq][F] fp32 stats of
    the unit's layer.  Returns (raw [Hq][n], agg [Hkv][n], kept list per KV head).
    """
    Hkv, n, d = k_bits.shape
    Hq = Hkv * group
    pos = np.asarray(pos)
    mu = np.asarray(q_mean_re, np.float64) + 1j * np.asarray(q_mean_im, np.float64)
    raw = np.empty((Hq, n), np.float64)
    for h in range(Hq):
        g = h // group
        p = pos if pos.ndim == 1 else pos[g]
        raw[h] = score_head(bf16_bits_to_f64(k_bits[g]), p, q_pos, mu[h], q_abs_mean[h],
                            head_dim, pairing, theta, offsets, form, reduce)
    a = aggregate_unit(raw, n, group, sink, window, agg)
    kept = [select(a[g], budget) for g in range(Hkv)]
    return raw, a, kept


def kth_threshold(agg: np.ndarray, n: int, budget: int, sink: int, window: int) -> float:
    """The smallest candidate aggregate that is kept (the B-th place), or +inf when
    nothing is dropped; used to judge slots whose order is decided by rounding."""
    prot = protected_mask(n, sink, window)
    cand = np.sort(agg[:n][~prot])[::-1]
    need = min(budget, n) - int(prot.sum())
    if need <= 0 or need > cand.size or min(budget, n) == n:
        return float("inf")
    return float(cand[need - 1])


# ----------------------------------------------------------------------------- calibration

def calibrate(q_bits: np.ndarray, pairing: str):
    """Calibrated query statistics of one (layer, query head) from T pre-RoPE query
    rows (bf16 bits [T][d]) [Calib issue, "How it works": per (layer, head, band)
    E[Re q_c[f]], E[Im q_c[f]], E|q_c[f]|, in the model's pairing layout; Blog, the
    calibration step: average the pre-RoPE queries per band].

    Returns (mean_re, mean_im, abs_mean, r, mrl), each [d/2] float64:
      r   = |E q_f| / E|q_f|            (0 where E|q_f| = 0): the concentration whose
            complement weighs the norm term [Blog, The Method: (1 - R_f)];
      mrl = |E[q_f / |q_f|]|            (q_f = 0 contributes 0): the circular mean
            resultant length of the band's phases [Blog: R = 1 when all point the
            same way, R = 0 when spread uniformly].
    """
    q = complex_bands(bf16_bits_to_f64(q_bits), pairing)          # [T][F]
    if q.shape[0] == 0:
        raise ValueError("no query rows")
    mean = q.mean(axis=0)
    mag = np.abs(q)
    abs_mean = mag.mean(axis=0)
    r = np.divide(np.abs(mean), abs_mean, out=np.zeros_like(abs_mean), where=abs_mean > 0)
    unit = np.divide(q, mag, out=np.zeros_like(q), where=mag > 0)
    mrl = np.abs(unit.mean(axis=0))
    return mean.real, mean.imag, abs_mean, r, mrl
