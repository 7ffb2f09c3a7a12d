"""Device-resident workloads for the C-ABI pass.

``DeviceProblem(cfg)`` uploads one synthetic workload (``synth.Config``) to the
GPU with torch (device memory and streams only), allocates every output and the
workspace, and runs the three entry points through the binding:
``score() -> select() -> compact()``.  All arithmetic runs in libtria.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as L
from . import synth


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def _bf16(arr: np.ndarray, device) -> torch.Tensor:
    """uint16 bf16 bit patterns -> a bf16 device tensor with the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16))
    return t.to(device).view(torch.bfloat16)


# Guard regions around every output buffer: GUARD elements before and after, filled
# with a canary the kernels never write, so that a write outside a buffer's extent
# shows up as a changed canary (check_guards).
GUARD = 2048
# canaries by element size, written through an integer view (for fp32: a NaN whose
# payload no kernel produces)
_CANARY = {1: 0xA5, 2: -0x5A5B, 4: 0x7FA5A5A5}
_INT_VIEW = {1: torch.uint8, 2: torch.int16, 4: torch.int32}


class Guarded:
    """Output tensors allocated inside larger buffers with canary-filled guards."""

    def __init__(self, device):
        self.device = device
        self.bufs = []

    def zeros(self, shape, dtype):
        n = 1
        for x in shape:
            n *= int(x)
        buf = torch.empty(n + 2 * GUARD, dtype=dtype, device=self.device)
        bits = buf.view(_INT_VIEW[buf.element_size()])
        bits.fill_(_CANARY[buf.element_size()])
        bits[GUARD:GUARD + n].zero_()
        self.bufs.append((bits, n))
        return buf[GUARD:GUARD + n].view(*shape)

    def check(self) -> None:
        for bits, n in self.bufs:
            c = _CANARY[bits.element_size()]
            if not (bool((bits[:GUARD] == c).all()) and bool((bits[GUARD + n:] == c).all())):
                raise AssertionError(f"a guard region of a {n}-element {bits.dtype} buffer was overwritten")


def params_for(cfg: synth.Config) -> L.TriaParams:
    return L.make_params(cfg.head_dim, cfg.n_kv_heads, cfg.group, cfg.n_layers,
                         L.PAIR_NEOX if cfg.pairing == "neox" else L.PAIR_INTERLEAVED,
                         L.AGG_MEAN if cfg.agg == "mean" else L.AGG_MAX,
                         cfg.rope_base, cfg.offsets, cfg.sink, cfg.window,
                         L.OFFSETS_MAX if cfg.offset_reduce == "max" else L.OFFSETS_MEAN)


def host_cache(cfg: synth.Config, which: str, workers: int | None = None) -> np.ndarray:
    """The K (``"k"``) or V (``"v"``) cache of a workload as bf16 bits, in the layout the
    device holds it: a paged pool, or dense [U][Hkv][n_max][d] padded to n_max slots
    (n_max = the longest unit rounded up to 16)."""
    if cfg.paged:
        return synth.build_cache(cfg, which, workers)
    n_max = round_up(max(synth.units(cfg).n_max, 1), 16)
    out = np.zeros((cfg.n_units, cfg.n_kv_heads, n_max, cfg.head_dim), dtype=np.uint16)
    for unit, head, rows in synth.iter_chunks(cfg, which, workers):
        out[unit, head, :rows.shape[0]] = rows
    return out


class DeviceProblem:
    """One workload resident in HBM, plus its outputs and workspace."""

    def __init__(self, cfg: synth.Config, device: str = "cuda:0", keep_raw: bool = True,
                 workers: int | None = None, k_host: np.ndarray | None = None, v_host: np.ndarray | None = None):
        self.cfg = cfg
        self.dev = torch.device(device)
        u = synth.units(cfg)
        self.units = u
        U, Hkv, G, d = cfg.n_units, cfg.n_kv_heads, cfg.group, cfg.head_dim
        self.n_max = round_up(max(u.n_max, 1), 16)
        self.b_max = max(u.b_max, 1)
        self.params = params_for(cfg)

        # --- K / V caches
        if k_host is None:
            k_host = self._host_cache("k", workers)
        self.K = _bf16(k_host, self.dev)
        del k_host
        if v_host is None:
            v_host = self._host_cache("v", workers)
        self.V = _bf16(v_host, self.dev)
        del v_host

        self.guards = Guarded(self.dev)
        gz = self.guards.zeros
        if cfg.paged:
            pg = synth.paging(cfg)
            self.paging = pg
            self.bt = torch.from_numpy(pg.block_table).to(self.dev)
            self.dbt = torch.from_numpy(pg.dst_block_table).to(self.dev)
            bs = cfg.block_size
            self.k_view = L.make_view(self.K, 0, d, Hkv * d, self.bt, bs, pg.block_table.shape[1], pg.n_blocks)
            self.v_view = L.make_view(self.V, 0, d, Hkv * d, self.bt, bs, pg.block_table.shape[1], pg.n_blocks)
            self.K_out = gz((pg.n_dst_blocks, bs, Hkv, d), torch.bfloat16)
            self.V_out = gz((pg.n_dst_blocks, bs, Hkv, d), torch.bfloat16)
            mdb = pg.dst_block_table.shape[1]
            self.kd_view = L.make_view(self.K_out, 0, d, Hkv * d, self.dbt, bs, mdb, pg.n_dst_blocks)
            self.vd_view = L.make_view(self.V_out, 0, d, Hkv * d, self.dbt, bs, mdb, pg.n_dst_blocks)
        else:
            self.paging = None
            nm = self.K.shape[2]
            self.k_view = L.make_view(self.K, Hkv * nm * d, nm * d, d)
            self.v_view = L.make_view(self.V, Hkv * nm * d, nm * d, d)
            self.K_out = gz((U, Hkv, self.b_max, d), torch.bfloat16)
            self.V_out = gz((U, Hkv, self.b_max, d), torch.bfloat16)
            self.kd_view = L.make_view(self.K_out, Hkv * self.b_max * d, self.b_max * d, d)
            self.vd_view = L.make_view(self.V_out, Hkv * self.b_max * d, self.b_max * d, d)

        # --- per-unit metadata and statistics
        to = lambda a, dt=torch.int32: torch.from_numpy(np.array(a, copy=True)).to(self.dev, dt)
        self.len = to(u.lengths)
        self.unit_layer = to(u.unit_layer)
        self.q_pos = to(u.q_pos)
        self.budget = to(u.budget)
        re, im, ab = synth.q_stats(cfg)
        self.q_re, self.q_im, self.q_abs = to(re, torch.float32), to(im, torch.float32), to(ab, torch.float32)
        pos = synth.positions_all(cfg)
        pos_pad = np.zeros((U, 1, self.n_max), np.int32)
        pos_pad[:, 0, :pos.shape[1]] = pos
        self.pos = to(pos_pad)

        # --- outputs and workspace
        Hq = cfg.n_q_heads
        self.raw = gz((U, Hq, self.n_max), torch.float32) if keep_raw else None
        self.agg = gz((U, Hkv, self.n_max), torch.float32)
        self.idx = gz((U, Hkv, self.b_max), torch.int32)
        self.cnt = gz((U,), torch.int32)
        self.pos_out = gz((U, Hkv, self.b_max), torch.int32)
        self.ws_bytes = L.tria_workspace_size(self.params, U, self.n_max)
        self.ws = gz((self.ws_bytes,), torch.uint8)

    def _host_cache(self, which: str, workers) -> np.ndarray:
        return host_cache(self.cfg, which, workers)

    # ------------------------------------------------------------------ the pass
    def score(self, stream=None):
        L.tria_score(self.params, self.k_view, self.cfg.n_units, self.n_max, self.len, self.unit_layer, self.q_pos,
                     self.q_re, self.q_im, self.q_abs, self.raw, self.agg, self.ws, self.ws_bytes, stream)

    def select(self, stream=None):
        L.tria_select(self.params, self.cfg.n_units, self.n_max, self.b_max, self.len, self.budget, self.agg,
                      self.idx, self.cnt, self.ws, self.ws_bytes, stream)

    def compact(self, idx=None, stream=None):
        L.tria_compact(self.params, self.k_view, self.v_view, self.pos, 1, self.cfg.n_units, self.n_max,
                       self.b_max, self.len, self.idx if idx is None else idx, self.cnt, self.kd_view, self.vd_view,
                       self.pos_out, stream)

    def run(self, stream=None):
        self.score(stream)
        self.select(stream)
        self.compact(stream=stream)

    def flags(self) -> int:
        return L.tria_device_flags(self.ws, torch.cuda.current_stream(self.dev))

    def check_guards(self) -> None:
        """Raises if a kernel wrote outside any output buffer (or the workspace)."""
        self.guards.check()

    # ------------------------------------------------------------------ readback helpers
    def kept(self, unit: int, kv_head: int) -> np.ndarray:
        k = int(self.cnt[unit].item())
        return self.idx[unit, kv_head, :k].cpu().numpy().astype(np.int64)

    def out_rows(self, which: str, unit: int, kv_head: int, count: int) -> np.ndarray:
        """bf16 bits [count][d] of the compacted rows of (unit, kv_head)."""
        T = self.K_out if which == "k" else self.V_out
        if not self.cfg.paged:
            t = T[unit, kv_head, :count]
        else:
            bs = self.cfg.block_size
            bt = torch.from_numpy(self.paging.dst_block_table[unit]).to(self.dev).long()
            j = torch.arange(count, device=self.dev)
            t = T[bt[j // bs], j % bs, kv_head]
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def algorithmic_bytes(self) -> int:
        """Bytes the pass must move at minimum: every K row read once, plus the kept K and V
        rows read and written, plus 4 B read + 4 B written of position per kept row."""
        cfg, u = self.cfg, self.units
        row = 2 * cfg.head_dim
        keys = int(u.lengths.astype(np.int64).sum()) * cfg.n_kv_heads
        kept = int(np.minimum(u.budget, u.lengths).astype(np.int64).sum()) * cfg.n_kv_heads
        return keys * row + kept * (4 * row + 8)

    def head_keys(self) -> int:
        return int(self.units.lengths.astype(np.int64).sum()) * self.cfg.n_kv_heads


def calibrate(params: L.TriaParams, q: torch.Tensor, want_r: bool = True, want_mrl: bool = True,
              stream=None) -> dict:
    """tria_calibrate over a device tensor q [L][Hq][T][d] (bf16 or its 16-bit pattern;
    any strides that are multiples of 8 elements, unit stride along d).  Allocates the
    outputs and the workspace; returns {"q_mean_re", "q_mean_im", "q_abs_mean", "r",
    "mrl"} as fp32 [L][Hq][d/2] device tensors (r, mrl None when not wanted)."""
    if q.dim() != 4 or q.element_size() != 2 or q.stride(3) != 1:
        raise ValueError("q must be a 16-bit [L][Hq][T][d] tensor with unit stride along d")
    Ln, Hq, T, d = q.shape
    F = d // 2
    dev = q.device
    out = {k: torch.empty((Ln, Hq, F), dtype=torch.float32, device=dev)
           for k in ("q_mean_re", "q_mean_im", "q_abs_mean")}
    out["r"] = torch.empty((Ln, Hq, F), dtype=torch.float32, device=dev) if want_r else None
    out["mrl"] = torch.empty((Ln, Hq, F), dtype=torch.float32, device=dev) if want_mrl else None
    ws_bytes = L.tria_calibrate_workspace_size(params, T)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    L.tria_calibrate(params, q, q.stride(0), q.stride(1), q.stride(2), T, out["q_mean_re"], out["q_mean_im"],
                     out["q_abs_mean"], out["r"], out["mrl"], ws, ws_bytes, stream)
    return out
