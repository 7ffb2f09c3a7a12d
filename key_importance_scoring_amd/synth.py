"""Seeded synthetic inputs for the TriAttention pruning pass.

These generators feed both the fp64 CPU oracle (under ``oracle/``) and the HIP
path, so they hold none of the method's arithmetic: no scoring, no offset
average, no normalisation, no selection, no compaction.  They only draw random
numbers, apply the ordinary rotary position embedding a model applies to a key
before it is cached (RoFormer's rotation, standard outside this method), and
round to bf16.

Recipe (the same for every workload, see ``CONFIGS``):

* key centre per (layer, KV head, band): ``c = r e^{i psi}``, ``r ~ U(0.5, 2)``,
  ``psi ~ U[0, 2 pi)``;  "non-concentrated" heads get ``r = 0``;
* pre-rotation key band ``k_f = c_f + (x + i y)``, ``x, y ~ N(0, 0.3^2)`` (the std
  is ``key_noise``, 0.3 in every workload);
* the key is rotated at its position ``p`` (band f turned by ``p * theta^(-2f/d)``),
  laid out in the model's pairing (NEOX: re in dims ``[0, d/2)``, im in
  ``[d/2, d)``; interleaved: re in even dims, im in odd dims) and rounded to
  bf16 (fp64 -> fp32 -> bf16, round-to-nearest-even at each step);
* values: ``N(0, 1)`` rounded to bf16 (their content never affects the pass);
* query statistics per (layer, q-head, band): centre ``mu`` drawn like the key
  centre, ``E|q_f| = |mu_f| (1 + U(0, 0.5))``, stored as fp32; for the q-heads
  of a non-concentrated KV head ``mu`` is scaled by 1e-3 while ``E|q_f|`` keeps
  an O(1) magnitude ``r (1 + U(0, 0.5))``, ``r ~ U(0.5, 2)``; ``mu_scale`` (1 in
  every workload) scales the other heads' ``mu`` after ``E|q_f|`` is drawn;
* positions are ``0 .. len-1`` (a fresh cache) and the current query sits at
  ``len - 1``.

Every draw is keyed by ``SeedSequence([seed, config id, stream kind, a, b])`` so
any (unit, head) chunk can be regenerated alone.
"""
from __future__ import annotations

import dataclasses
import functools
import math
import os
from dataclasses import dataclass, field

import numpy as np

# stream kinds for SeedSequence
_K_CENTRE, _K_NOISE, _V_ROWS, _Q_STATS, _LENGTHS, _BLOCKS, _NONCONC, _Q_ROWS, _DEC_K, _DEC_V = range(10)


@dataclass(frozen=True)
class Config:
    """One synthetic workload.  A *unit* is one (layer, sequence) pair."""
    name: str
    cid: int
    n_layers: int
    n_kv_heads: int
    group: int
    head_dim: int
    pairing: str            # "neox" | "interleaved"
    rope_base: float
    n_kv: int               # keys per unit (dense) or the largest length (ragged)
    offsets: tuple
    window: int
    sink: int
    agg: str                # "mean" | "max"
    budget: int = 0         # absolute budget per unit (used when budget_frac == 0)
    budget_frac: float = 0.0  # budget = floor(len * frac) when > 0
    n_seqs: int = 1
    ragged_min: int = 0     # > 0: lengths ~ U{ragged_min .. n_kv}
    paged: bool = False
    block_size: int = 16
    nonconc_frac: float = 0.0
    seed: int = 0
    offset_reduce: str = "mean"   # "mean" (the method) | "max": reduction over the future offsets
    key_noise: float = 0.3        # std of each pre-rotation key component around the centre
    mu_scale: float = 1.0         # scales the query centres E[q_f] only (E|q_f| is drawn unscaled)

    @property
    def n_q_heads(self) -> int:
        return self.n_kv_heads * self.group

    @property
    def n_units(self) -> int:
        return self.n_layers * self.n_seqs

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


def _geom(k: int) -> tuple:
    return tuple(2 ** i for i in range(k))


CONFIGS = {
    "tiny": Config(
        name="tiny", cid=0, n_layers=1, n_kv_heads=2, group=4, head_dim=64,
        pairing="neox", rope_base=1e4, n_kv=2048, offsets=_geom(13),
        budget=1024, window=256, sink=0, agg="mean"),
    "qwen3_8b": Config(
        name="qwen3_8b", cid=1, n_layers=36, n_kv_heads=8, group=4, head_dim=128,
        pairing="neox", rope_base=1e6, n_kv=32768, offsets=_geom(17),
        budget=2048, window=128, sink=4, agg="max"),
    "qwen3_32b": Config(
        name="qwen3_32b", cid=2, n_layers=64, n_kv_heads=8, group=8, head_dim=128,
        pairing="neox", rope_base=1e6, n_kv=32768, offsets=_geom(17),
        budget=12000, window=256, sink=0, agg="mean", nonconc_frac=0.1),
    "batched_decode": Config(
        name="batched_decode", cid=3, n_layers=1, n_kv_heads=8, group=4, head_dim=128,
        pairing="neox", rope_base=1e6, n_kv=32768, offsets=_geom(17),
        budget_frac=0.5, window=256, sink=0, agg="max", n_seqs=64,
        ragged_min=4096, paged=True, block_size=16),
    "long_context": Config(
        name="long_context", cid=4, n_layers=1, n_kv_heads=8, group=8, head_dim=128,
        pairing="interleaved", rope_base=1e6, n_kv=131072, offsets=_geom(17),
        budget=13107, window=512, sink=4, agg="max"),
}


def _rng(cfg: Config, kind: int, a: int = 0, b: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg.seed, cfg.cid, kind, a, b]))


# --------------------------------------------------------------------------- bf16

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns the uint16 bit pattern."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


# --------------------------------------------------------------------------- units

@dataclass
class Units:
    lengths: np.ndarray      # int32 [U]
    unit_layer: np.ndarray   # int32 [U]
    unit_seq: np.ndarray     # int32 [U]
    q_pos: np.ndarray        # int32 [U]
    budget: np.ndarray       # int32 [U]
    n_max: int
    b_max: int               # largest number of kept rows in any unit


@functools.lru_cache(maxsize=16)
def units(cfg: Config) -> Units:
    """Per-unit metadata.  Unit u = layer * n_seqs + seq."""
    if cfg.ragged_min > 0:
        seq_len = _rng(cfg, _LENGTHS).integers(cfg.ragged_min, cfg.n_kv, size=cfg.n_seqs,
                                               endpoint=True).astype(np.int32)
    else:
        seq_len = np.full(cfg.n_seqs, cfg.n_kv, dtype=np.int32)
    lengths = np.tile(seq_len, cfg.n_layers).astype(np.int32)
    unit_layer = np.repeat(np.arange(cfg.n_layers, dtype=np.int32), cfg.n_seqs)
    unit_seq = np.tile(np.arange(cfg.n_seqs, dtype=np.int32), cfg.n_layers)
    if cfg.budget_frac > 0:
        budget = np.floor(lengths.astype(np.float64) * cfg.budget_frac).astype(np.int32)
    else:
        budget = np.full(cfg.n_units, cfg.budget, dtype=np.int32)
    q_pos = (lengths - 1).astype(np.int32)
    n_max = int(lengths.max())
    b_max = int(np.minimum(budget, lengths).max())
    for a in (lengths, unit_layer, unit_seq, q_pos, budget):
        a.setflags(write=False)
    return Units(lengths, unit_layer, unit_seq, q_pos, budget, n_max, b_max)


def positions(cfg: Config, unit: int) -> np.ndarray:
    """Positions of the cached slots of one unit (fresh cache: 0 .. len-1)."""
    return np.arange(int(units(cfg).lengths[unit]), dtype=np.int32)


# --------------------------------------------------------------------------- heads

@functools.lru_cache(maxsize=16)
def nonconcentrated(cfg: Config) -> np.ndarray:
    """bool [L][Hkv]: (layer, KV head) pairs whose keys have no centre."""
    mask = np.zeros((cfg.n_layers, cfg.n_kv_heads), dtype=bool)
    total = cfg.n_layers * cfg.n_kv_heads
    k = int(round(cfg.nonconc_frac * total))
    if k > 0:
        pick = _rng(cfg, _NONCONC).permutation(total)[:k]
        mask.reshape(-1)[pick] = True
    mask.setflags(write=False)
    return mask


def _centre(rng: np.random.Generator, n: int) -> np.ndarray:
    r = rng.uniform(0.5, 2.0, size=n)
    psi = rng.uniform(0.0, 2.0 * math.pi, size=n)
    return r * np.exp(1j * psi)


def key_centres(cfg: Config, layer: int, kv_head: int) -> np.ndarray:
    """complex128 [F]: the pre-rotation key centre of one (layer, KV head)."""
    F = cfg.head_dim // 2
    c = _centre(_rng(cfg, _K_CENTRE, layer, kv_head), F)
    if nonconcentrated(cfg)[layer, kv_head]:
        c = np.zeros_like(c)
    return c


@functools.lru_cache(maxsize=8)
def q_stats(cfg: Config):
    """(q_mean_re, q_mean_im, q_abs_mean), each float32 [L][Hq][F] (read-only)."""
    F = cfg.head_dim // 2
    L, Hq = cfg.n_layers, cfg.n_q_heads
    re = np.zeros((L, Hq, F), np.float32)
    im = np.zeros((L, Hq, F), np.float32)
    ab = np.zeros((L, Hq, F), np.float32)
    nc = nonconcentrated(cfg)
    for l in range(L):
        for h in range(Hq):
            rng = _rng(cfg, _Q_STATS, l, h)
            mu = _centre(rng, F)
            spread = 1.0 + rng.uniform(0.0, 0.5, size=F)
            if nc[l, h // cfg.group]:
                r = rng.uniform(0.5, 2.0, size=F)
                absm = r * spread
                mu = mu * 1e-3
            else:
                absm = np.abs(mu) * spread
                mu = mu * cfg.mu_scale
            re[l, h] = mu.real
            im[l, h] = mu.imag
            ab[l, h] = absm
    for x in (re, im, ab):
        x.setflags(write=False)
    return re, im, ab


# --------------------------------------------------------------------------- rows

@functools.lru_cache(maxsize=4)
def _rotation(n: int, head_dim: int, base: float):
    """cos/sin tables [n][F] of the standard rotary embedding at positions 0..n-1."""
    F = head_dim // 2
    inv_freq = base ** (-(2.0 * np.arange(F, dtype=np.float64)) / head_dim)
    ang = np.outer(np.arange(n, dtype=np.float64), inv_freq)
    return np.cos(ang), np.sin(ang)


def _layout(re: np.ndarray, im: np.ndarray, pairing: str) -> np.ndarray:
    n, F = re.shape
    out = np.empty((n, 2 * F), dtype=np.float64)
    if pairing == "neox":
        out[:, :F] = re
        out[:, F:] = im
    elif pairing == "interleaved":
        out[:, 0::2] = re
        out[:, 1::2] = im
    else:
        raise ValueError(pairing)
    return out


def key_rows(cfg: Config, unit: int, kv_head: int) -> np.ndarray:
    """uint16 [len][d]: bf16 bits of the cached (rotated) keys of one (unit, KV head)."""
    u = units(cfg)
    n = int(u.lengths[unit])
    layer = int(u.unit_layer[unit])
    F = cfg.head_dim // 2
    c = key_centres(cfg, layer, kv_head)
    rng = _rng(cfg, _K_NOISE, unit, kv_head)
    noise = rng.standard_normal((2, n, F)) * cfg.key_noise
    a = c.real[None, :] + noise[0]
    b = c.imag[None, :] + noise[1]
    cos, sin = _rotation(cfg.n_kv, cfg.head_dim, cfg.rope_base)
    cos, sin = cos[:n], sin[:n]
    ra = a * cos - b * sin
    rb = a * sin + b * cos
    return f32_to_bf16_bits(_layout(ra, rb, cfg.pairing).astype(np.float32))


def decode_rows(cfg: Config, unit: int, kv_head: int, p0: int, count: int, which: str) -> np.ndarray:
    """uint16 [count][d]: bf16 bits of the keys (``"k"``) or values (``"v"``) that a
    decode loop appends for the tokens at positions p0 .. p0 + count - 1 of one
    (unit, KV head).  Keys are drawn like the cache's (the (layer, KV head) centre
    plus N(0, 0.3^2) per component, rotated at their positions), values N(0, 1);
    each chunk is seeded by (unit, KV head, p0), so a chunk can be redrawn alone."""
    F = cfg.head_dim // 2
    if which == "v":
        rng = _rng(cfg, _DEC_V, unit * 4096 + kv_head, p0)
        return f32_to_bf16_bits(rng.standard_normal((count, cfg.head_dim), dtype=np.float32))
    layer = int(units(cfg).unit_layer[unit])
    c = key_centres(cfg, layer, kv_head)
    rng = _rng(cfg, _DEC_K, unit * 4096 + kv_head, p0)
    noise = rng.standard_normal((2, count, F)) * cfg.key_noise
    a = c.real[None, :] + noise[0]
    b = c.imag[None, :] + noise[1]
    inv_freq = cfg.rope_base ** (-(2.0 * np.arange(F, dtype=np.float64)) / cfg.head_dim)
    ang = np.outer(np.arange(p0, p0 + count, dtype=np.float64), inv_freq)
    cos, sin = np.cos(ang), np.sin(ang)
    return f32_to_bf16_bits(_layout(a * cos - b * sin, a * sin + b * cos, cfg.pairing).astype(np.float32))


def query_rows(cfg: Config, layer: int, q_head: int, n_tokens: int) -> np.ndarray:
    """uint16 [n_tokens][d]: bf16 bits of a synthetic stream of pre-RoPE queries of one
    (layer, query head), the input of calibration: each band is the head's centre
    (the E[q_f] of q_stats) plus N(0, 0.3^2) per component, laid out per the pairing."""
    re, im, _ = q_stats(cfg)
    F = cfg.head_dim // 2
    rng = _rng(cfg, _Q_ROWS, layer, q_head)
    noise = rng.standard_normal((2, n_tokens, F)) * 0.3
    a = re[layer, q_head][None, :].astype(np.float64) + noise[0]
    b = im[layer, q_head][None, :].astype(np.float64) + noise[1]
    return f32_to_bf16_bits(_layout(a, b, cfg.pairing).astype(np.float32))


def _query_job(args):
    cfg, layer, q_head, n_tokens = args
    return layer, q_head, query_rows(cfg, layer, q_head, n_tokens)


def query_stream(cfg: Config, n_tokens: int, workers: int | None = None) -> np.ndarray:
    """uint16 [L][Hq][n_tokens][d]: query_rows of every (layer, query head); drawn in a
    process pool as iter_chunks does."""
    out = np.empty((cfg.n_layers, cfg.n_q_heads, n_tokens, cfg.head_dim), np.uint16)
    jobs = [(cfg, l, h, n_tokens) for l in range(cfg.n_layers) for h in range(cfg.n_q_heads)]
    for l, h, rows in _run_jobs(_query_job, jobs, workers):
        out[l, h] = rows
    return out


def value_rows(cfg: Config, unit: int, kv_head: int) -> np.ndarray:
    """uint16 [len][d]: bf16 bits of the cached values of one (unit, KV head)."""
    n = int(units(cfg).lengths[unit])
    rng = _rng(cfg, _V_ROWS, unit, kv_head)
    return f32_to_bf16_bits(rng.standard_normal((n, cfg.head_dim), dtype=np.float32))


# --------------------------------------------------------------------------- paging

@dataclass
class Paging:
    block_table: np.ndarray   # int32 [U][max_blocks], -1 past the end
    n_blocks: int
    dst_block_table: np.ndarray  # int32 [U][max_dst_blocks], -1 past the end
    n_dst_blocks: int


@functools.lru_cache(maxsize=16)
def paging(cfg: Config) -> Paging:
    """Shuffled block tables for the source cache and for the compacted cache."""
    u = units(cfg)
    bs = cfg.block_size

    def table(counts, kind):
        nb = int(sum(counts))
        perm = _rng(cfg, _BLOCKS, kind).permutation(nb).astype(np.int32)
        mb = int(max(counts)) if len(counts) else 0
        bt = np.full((len(counts), max(mb, 1)), -1, dtype=np.int32)
        off = 0
        for i, c in enumerate(counts):
            bt[i, :c] = perm[off:off + c]
            off += c
        return bt, nb

    src_counts = [(-(-int(n) // bs)) for n in u.lengths]
    kept = np.minimum(u.budget, u.lengths)
    dst_counts = [(-(-int(k) // bs)) for k in kept]
    bt, nb = table(src_counts, 0)
    dbt, dnb = table(dst_counts, 1)
    return Paging(bt, nb, dbt, dnb)


# --------------------------------------------------------------------------- whole caches

def _chunk_job(args):
    cfg, which, unit, head = args
    return (unit, head, key_rows(cfg, unit, head) if which == "k" else value_rows(cfg, unit, head))


def _jobs(cfg: Config, which: str):
    return [(cfg, which, u, g) for u in range(cfg.n_units) for g in range(cfg.n_kv_heads)]


def _run_jobs(fn, jobs, workers: int | None):
    """Yield fn(job) for every job, in a spawned process pool when workers > 1 (in an
    arbitrary order then).  workers = None: TRIA_SYNTH_WORKERS, else up to 16 processes
    for more than 16 jobs."""
    if workers is None:
        env = os.environ.get("TRIA_SYNTH_WORKERS")
        if env:
            workers = int(env)
        else:
            workers = min(16, os.cpu_count() or 1) if len(jobs) > 16 else 1
    if workers <= 1:
        for j in jobs:
            yield fn(j)
        return
    import multiprocessing as mp
    with mp.get_context("spawn").Pool(workers) as pool:
        for item in pool.imap_unordered(fn, jobs, chunksize=2):
            yield item


def iter_chunks(cfg: Config, which: str, workers: int | None = None):
    """Yield (unit, kv_head, rows) for every chunk of the K (``"k"``) or V (``"v"``) cache.

    With ``workers > 1`` the chunks are drawn in a spawned process pool (no GPU state
    is inherited); the order of the yielded chunks is then arbitrary.  The default
    pool size can be set with the environment variable TRIA_SYNTH_WORKERS (1 keeps
    everything in-process, e.g. under a profiler that attaches to every process).
    """
    yield from _run_jobs(_chunk_job, _jobs(cfg, which), workers)


def dense_shape(cfg: Config):
    u = units(cfg)
    return (cfg.n_units, cfg.n_kv_heads, u.n_max, cfg.head_dim)


def paged_shape(cfg: Config):
    pg = paging(cfg)
    return (pg.n_blocks, cfg.block_size, cfg.n_kv_heads, cfg.head_dim)


def place_chunk(cfg: Config, dest: np.ndarray, unit: int, kv_head: int, rows: np.ndarray,
                pg: Paging | None = None) -> None:
    """Write one (unit, KV head) chunk into a dense [U][Hkv][n_max][d] array or a paged
    [blocks][bs][Hkv][d] pool (through the source block table)."""
    n = rows.shape[0]
    if not cfg.paged:
        dest[unit, kv_head, :n] = rows
        return
    bs = cfg.block_size
    bt = pg.block_table[unit]
    slots = np.arange(n)
    dest[bt[slots // bs], slots % bs, kv_head] = rows


def build_cache(cfg: Config, which: str, workers: int | None = None) -> np.ndarray:
    """The whole K or V cache as bf16 bits (dense or paged, per ``cfg.paged``)."""
    pg = paging(cfg) if cfg.paged else None
    shape = paged_shape(cfg) if cfg.paged else dense_shape(cfg)
    out = np.zeros(shape, dtype=np.uint16)
    for unit, head, rows in iter_chunks(cfg, which, workers):
        place_chunk(cfg, out, unit, head, rows, pg)
    return out


def positions_all(cfg: Config) -> np.ndarray:
    """int32 [U][n_max]: slot positions (shared by all KV heads of a unit); 0 past len."""
    u = units(cfg)
    pos = np.zeros((cfg.n_units, u.n_max), dtype=np.int32)
    for i, n in enumerate(u.lengths):
        pos[i, :n] = np.arange(n, dtype=np.int32)
    return pos
