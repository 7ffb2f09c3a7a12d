"""GPU parity of the decode loop (tria_append, tria_compact_inplace, and the pass run
repeatedly on a cache that keeps per-head positions) against an oracle loop.

The oracle loop keeps, per (sequence, KV head), the positions and the K / V bits of
the slots it holds.  At every prune it scores them with the fp64 oracle using those
per-head positions (the kernels use only the newest position), checks the GPU's
aggregates and kept set (the tolerance rule of the single pass), then adopts the
GPU's kept set, so that both stay in step; the compacted rows and positions must
then match bit for bit.  In-place compaction is also checked against the
out-of-place tria_compact on the same indices.
"""
import numpy as np
import pytest
import torch

from _parity import check_agg, check_kept, log
from oracle import tria_oracle as o
from key_importance_scoring_amd import _lib as L
from key_importance_scoring_amd import synth
from key_importance_scoring_amd.decode import DecodeLoop

pytestmark = pytest.mark.gpu

C = synth.CONFIGS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    L.load()


CASES = {
    # budget, interval, steps
    "bd_neox": (C["batched_decode"].replace(name="dec_neox", n_seqs=3, n_kv_heads=2, window=64, sink=2), 300, 128, 7),
    "lc_inter_g8": (C["long_context"].replace(name="dec_inter", n_kv_heads=2, window=100, sink=4, paged=True,
                                              block_size=16), 400, 128, 6),
    "d64_bs7_max": (C["tiny"].replace(name="dec_d64", n_seqs=2, paged=True, block_size=7, window=32, sink=0,
                                      offset_reduce="max"), 200, 96, 6),
}


def _stats(cfg):
    re, im, ab = synth.q_stats(cfg)
    return re.astype(np.float64) + 1j * im.astype(np.float64), ab.astype(np.float64)


def _drive(loop, cfg, budget, interval, steps, pairs, name):
    """Runs the loop for `steps` appends and, after every prune, checks the
    (sequence, KV head) pairs in `pairs` against the oracle loop; returns the number
    of prunes checked."""
    mu, absm = _stats(cfg)
    layer = synth.units(cfg).unit_layer
    G = cfg.group
    # oracle state per (sequence, KV head): positions, K bits, V bits
    st = {(u, g): (np.zeros(0, np.int64), np.zeros((0, cfg.head_dim), np.uint16),
                   np.zeros((0, cfg.head_dim), np.uint16)) for u, g in pairs}
    checked = 0
    for step in range(steps):
        kn, vn, pn = loop.new_rows(interval)
        for (u, g), (ps, ks, vs) in st.items():
            st[(u, g)] = (np.concatenate([ps, pn[u]]), np.concatenate([ks, kn[u, g]]), np.concatenate([vs, vn[u, g]]))
        pruned = loop.step(rows=(kn, vn, pn))
        torch.cuda.synchronize()
        assert loop.flags() == 0
        loop.check_guards()
        # the library advanced the device state: lengths (append, then the kept
        # count after a prune) and the newest position as the query position
        np.testing.assert_array_equal(loop.len.cpu().numpy(), loop.len_host)
        np.testing.assert_array_equal(loop.q_pos.cpu().numpy(), loop.next_pos - 1)
        if not pruned:
            continue
        checked += 1
        q_pos = int(loop.next_pos[0] - 1)
        agg = loop.agg.cpu().numpy()
        idx = loop.idx.cpu().numpy()
        cnt = loop.cnt.cpu().numpy()
        for (u, g), (ps, ks, vs) in list(st.items()):
            n = ps.size
            what = f"{name} step {step} seq {u} kv {g}"
            rows = o.bf16_bits_to_f64(ks)
            raw = np.stack([o.score_head(rows, ps, q_pos, mu[layer[u], h], absm[layer[u], h], cfg.head_dim,
                                         cfg.pairing, cfg.rope_base, cfg.offsets, "direct", cfg.offset_reduce)
                            for h in range(g * G, (g + 1) * G)])
            o_agg = o.aggregate_unit(raw, n, G, cfg.sink, cfg.window, cfg.agg)[0]
            o_kept = o.select(o_agg, budget)
            check_agg(agg[u, g, :n], o_agg, what)
            k = int(cnt[u])
            assert k == min(budget, n), what
            g_kept = idx[u, g, :k].astype(np.int64)
            check_kept(g_kept, o_kept, o_agg, n, budget, cfg.sink, cfg.window, what)
            # both continue from the GPU's kept set
            st[(u, g)] = (ps[g_kept], ks[g_kept], vs[g_kept])
        pos = loop.pos.cpu().numpy()
        for (u, g), (ps, ks, vs) in st.items():
            k = ps.size
            what = f"{name} step {step} seq {u} kv {g}"
            np.testing.assert_array_equal(pos[u, g, :k], ps, err_msg=what)
            np.testing.assert_array_equal(loop.head_rows("k", u, g, k), ks, err_msg=what)
            np.testing.assert_array_equal(loop.head_rows("v", u, g, k), vs, err_msg=what)
        # every pair: the kept count, ascending positions, the window's newest slots kept
        for u in range(cfg.n_units):
            k = int(cnt[u])
            assert k == min(budget, int(loop.len_host[u]))
            for g in range(cfg.n_kv_heads):
                assert (np.diff(pos[u, g, :k]) > 0).all(), (name, step, u, g)
                assert pos[u, g, k - 1] == loop.next_pos[u] - 1
    return checked


@pytest.mark.parametrize("name", list(CASES))
def test_decode_loop_matches_oracle_loop(name):
    cfg, budget, interval, steps = CASES[name]
    log(f"[decode] {name}: seqs={cfg.n_units} Hkv={cfg.n_kv_heads} G={cfg.group} d={cfg.head_dim} "
        f"budget={budget} interval={interval} bs={cfg.block_size} reduce={cfg.offset_reduce}")
    loop = DecodeLoop(cfg, budget, interval)
    pairs = [(u, g) for u in range(cfg.n_units) for g in range(cfg.n_kv_heads)]
    assert _drive(loop, cfg, budget, interval, steps, pairs, name) >= 2


def test_decode_loop_full_size_sampled():
    """The benchmark's decode loop (64 sequences x 8 KV heads, d 128, G 4, paged,
    budget 2048, window 256, sink 0, interval 128) through three prunes: sampled
    (sequence, KV head) pairs against the oracle loop, properties on every pair."""
    cfg = C["batched_decode"].replace(name="decode_loop", n_seqs=64, ragged_min=0, window=256, sink=0)
    budget, interval = 2048, 128
    log(f"[decode] full size: seqs={cfg.n_units} Hkv={cfg.n_kv_heads} budget={budget}")
    loop = DecodeLoop(cfg, budget, interval)
    steps = -(-budget // interval) + 3
    assert _drive(loop, cfg, budget, interval, steps, [(0, 0), (37, 5), (63, 7)], "decode_full") == 3


def test_inplace_matches_out_of_place():
    """tria_compact_inplace on a paged cache gives what tria_compact gives into a
    separate cache, for random ascending kept sets (rows that stay, runs that move,
    a budget above the length)."""
    cfg = C["batched_decode"].replace(name="inplace", n_seqs=4, n_kv_heads=3, block_size=16)
    U, Hkv, d, bs = cfg.n_units, cfg.n_kv_heads, cfg.head_dim, cfg.block_size
    n_max, b_max = 1024, 700
    rng = np.random.default_rng(5)
    lens = np.array([1024, 900, 300, 1], np.int32)
    nb = n_max // bs
    table = rng.permutation(U * nb).astype(np.int32).reshape(U, nb)
    k_bits = rng.integers(0, 1 << 16, size=(U * nb, bs, Hkv, d), dtype=np.uint16)
    v_bits = rng.integers(0, 1 << 16, size=(U * nb, bs, Hkv, d), dtype=np.uint16)
    idx = np.full((U, Hkv, b_max), -1, np.int32)
    cnt = np.minimum(lens, b_max).astype(np.int32)
    for u in range(U):
        for g in range(Hkv):
            keep = np.sort(rng.choice(int(lens[u]), size=int(cnt[u]), replace=False))
            keep[: min(5, keep.size)] = np.arange(min(5, keep.size))        # a prefix that stays
            idx[u, g, :cnt[u]] = np.unique(keep) if np.unique(keep).size == cnt[u] else np.arange(cnt[u])
    pos = rng.integers(0, 1 << 20, size=(U, Hkv, n_max)).astype(np.int32)
    dev = "cuda:0"
    p = L.make_params(d, Hkv, cfg.group, 1, L.PAIR_NEOX, L.AGG_MAX, 1e6, [1], 0, 0)
    t = lambda a: torch.from_numpy(a).to(dev)
    K = t(k_bits.view(np.int16))
    V = t(v_bits.view(np.int16))
    bt = t(table)
    kv = L.make_view(K, 0, d, Hkv * d, bt, bs, nb, U * nb)
    vv = L.make_view(V, 0, d, Hkv * d, bt, bs, nb, U * nb)
    ws = torch.zeros(256, dtype=torch.uint8, device=dev)
    # out of place first (into dense buffers), from the untouched cache
    Kd = torch.zeros((U, Hkv, b_max, d), dtype=torch.int16, device=dev)
    Vd = torch.zeros_like(Kd)
    Pd = torch.zeros((U, Hkv, b_max), dtype=torch.int32, device=dev)
    kdv = L.make_view(Kd, Hkv * b_max * d, b_max * d, d)
    vdv = L.make_view(Vd, Hkv * b_max * d, b_max * d, d)
    P = t(pos)
    L.tria_compact(p, kv, vv, P, Hkv, U, n_max, b_max, t(lens), t(idx), t(cnt), kdv, vdv, Pd)
    lens_d = t(lens)
    L.tria_compact_inplace(p, kv, vv, P, U, n_max, b_max, lens_d, t(idx), t(cnt), ws)
    torch.cuda.synchronize()
    assert L.tria_device_flags(ws) == 0
    np.testing.assert_array_equal(lens_d.cpu().numpy(), cnt)          # len <- the kept count
    Kh, Vh, Ph = K.cpu().numpy(), V.cpu().numpy(), P.cpu().numpy()
    Kdh, Vdh, Pdh = Kd.cpu().numpy(), Vd.cpu().numpy(), Pd.cpu().numpy()
    for u in range(U):
        k = int(cnt[u])
        slots = np.arange(k)
        for g in range(Hkv):
            np.testing.assert_array_equal(Kh[table[u, slots // bs], slots % bs, g], Kdh[u, g, :k])
            np.testing.assert_array_equal(Vh[table[u, slots // bs], slots % bs, g], Vdh[u, g, :k])
            np.testing.assert_array_equal(Ph[u, g, :k], Pdh[u, g, :k])
            # slots past the kept count are untouched
            rest = np.arange(k, int(lens[u]))
            np.testing.assert_array_equal(Kh[table[u, rest // bs], rest % bs, g],
                                          k_bits.view(np.int16)[table[u, rest // bs], rest % bs, g])


def test_inplace_flags_descending_indices():
    """An index list that is not ascending cannot be compacted in place: it is flagged
    and the offending rows are left where they are (no other row is touched)."""
    d, Hkv, n_max, b_max = 64, 1, 64, 8
    dev = "cuda:0"
    p = L.make_params(d, Hkv, 1, 1, L.PAIR_NEOX, L.AGG_MAX, 1e6, [1], 0, 0)
    K = torch.arange(n_max * d, dtype=torch.int32, device=dev).to(torch.int16).reshape(1, 1, n_max, d)
    V = K.clone() + 1
    k0, v0 = K.clone(), V.clone()
    kv = L.make_view(K, n_max * d, n_max * d, d)
    vv = L.make_view(V, n_max * d, n_max * d, d)
    idx = torch.tensor([[[0, 1, 9, 5, 20, 21, 22, 23]]], dtype=torch.int32, device=dev)
    ws = torch.zeros(256, dtype=torch.uint8, device=dev)
    lens_d = torch.tensor([40], dtype=torch.int32, device=dev)
    L.tria_compact_inplace(p, kv, vv, None, 1, n_max, b_max, lens_d, idx,
                           torch.tensor([8], dtype=torch.int32, device=dev), ws)
    torch.cuda.synchronize()
    assert int(lens_d[0]) == 8
    assert L.tria_device_flags(ws) & L.FLAG_INDEX
    # rows 0, 1 stay; row 2 <- row 9; row 3 (index 5 < 9) is left; rows 4.. <- 20..
    assert torch.equal(K[0, 0, 2], k0[0, 0, 9]) and torch.equal(K[0, 0, 3], k0[0, 0, 3])
    assert torch.equal(K[0, 0, 4], k0[0, 0, 20]) and torch.equal(V[0, 0, 7], v0[0, 0, 23])


def test_append_advances_len_and_query_position():
    """tria_append writes the rows at len[u] .., then len[u] <- min(len[u] + t, n_max)
    and q_pos[u] <- the newest position; rows that would land past n_max are skipped
    and flagged."""
    d, Hkv, U, n_max, t_new = 64, 2, 3, 64, 8
    dev = "cuda:0"
    p = L.make_params(d, Hkv, 1, 1, L.PAIR_NEOX, L.AGG_MAX, 1e6, [1], 0, 0)
    K = torch.zeros((U, Hkv, n_max, d), dtype=torch.int16, device=dev)
    V = torch.zeros_like(K)
    P = torch.full((U, Hkv, n_max), -1, dtype=torch.int32, device=dev)
    kv = L.make_view(K, Hkv * n_max * d, n_max * d, d)
    vv = L.make_view(V, Hkv * n_max * d, n_max * d, d)
    rng = np.random.default_rng(11)
    kn = torch.from_numpy(rng.integers(-30000, 30000, size=(U, Hkv, t_new, d), dtype=np.int16)).to(dev)
    vn = torch.from_numpy(rng.integers(-30000, 30000, size=(U, Hkv, t_new, d), dtype=np.int16)).to(dev)
    pn = torch.from_numpy((np.arange(U * t_new, dtype=np.int32) * 3 + 100).reshape(U, t_new)).to(dev)
    lens0 = np.array([0, 10, n_max - 5], np.int32)
    lens = torch.from_numpy(lens0.copy()).to(dev)
    q_pos = torch.zeros(U, dtype=torch.int32, device=dev)
    ws = torch.zeros(256, dtype=torch.uint8, device=dev)
    L.tria_append(p, kv, vv, P, U, n_max, lens, q_pos, t_new, kn, vn, pn, ws)
    torch.cuda.synchronize()
    assert L.tria_device_flags(ws) == L.FLAG_LEN                     # unit 2 runs past n_max
    np.testing.assert_array_equal(lens.cpu().numpy(), np.minimum(lens0 + t_new, n_max))
    np.testing.assert_array_equal(q_pos.cpu().numpy(), pn[:, -1].cpu().numpy())
    for u in range(U):
        fit = min(t_new, n_max - int(lens0[u]))
        sl = slice(int(lens0[u]), int(lens0[u]) + fit)
        assert torch.equal(K[u, :, sl], kn[u, :, :fit]) and torch.equal(V[u, :, sl], vn[u, :, :fit])
        for g in range(Hkv):
            assert torch.equal(P[u, g, sl], pn[u, :fit])
    assert (K[0, :, t_new:] == 0).all()                               # nothing past the new rows
