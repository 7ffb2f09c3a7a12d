#!/usr/bin/env python3
"""Throughput of the TriAttention pruning pass on one MI355X.

One step = tria_score -> tria_select -> tria_compact over the whole workload
(every layer, sequence and KV head), inputs resident in HBM.  Prints one JSON
line.  Default workload: Qwen3-8B-shaped, 36 layers x 8 KV heads x 32768 keys.

    python bench.py [--gpus 1] [--steps 50] [--warmup 100] [--config qwen3_8b]

The default line also carries the Qwen3-32B-shaped pass under "extra_workloads"
(--no-extra: the --config workload only).  With --read-probe GB it times the
streaming-read probe (the practical read ceiling) instead of the pass.

With --calibrate it times the calibration reduction instead (tria_calibrate over a
Qwen3-8B-shaped stream of 8192 pre-RoPE query rows per layer and query head) and
prints that measurement's JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "M keys scored+selected+compacted/s at n_kv=32K; % of HBM peak GB/s"
HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, published


def workload_desc(cfg) -> dict:
    d = {"workload": cfg.name, "layers": cfg.n_layers, "sequences": cfg.n_seqs, "kv_heads": cfg.n_kv_heads,
         "q_heads": cfg.n_q_heads, "head_dim": cfg.head_dim, "n_kv": cfg.n_kv, "pairing": cfg.pairing,
         "rope_base": cfg.rope_base, "offsets": len(cfg.offsets), "window": cfg.window, "sink": cfg.sink,
         "gqa": cfg.agg, "paged": cfg.paged, "offset_reduce": cfg.offset_reduce}
    if cfg.budget_frac:
        d["budget"] = f"{cfg.budget_frac:g} of each length"
    else:
        d["budget"] = cfg.budget
    if cfg.ragged_min:
        d["lengths"] = f"U{{{cfg.ragged_min}..{cfg.n_kv}}}"
    if cfg.nonconc_frac:
        d["nonconcentrated_heads"] = cfg.nonconc_frac
    return d


def _baseline_init():
    """Pool worker set-up: one BLAS thread per process (the pool spans the cores)."""
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _baseline_ready(_):
    from key_importance_scoring_amd import synth  # noqa: F401  (imports paid before the clock starts)
    from oracle import tria_oracle  # noqa: F401
    return os.getpid()


def _baseline_pairs(job):
    """One worker's share: the oracle on each (unit, KV head) of `pairs`, timed around
    the oracle's own steps only (input generation is outside the clock).  Returns
    (keys, oracle seconds, pairs)."""
    import numpy as np
    from key_importance_scoring_amd import synth
    from oracle import tria_oracle as o

    cfg, pairs, form = job
    u = synth.units(cfg)
    re, im, ab = synth.q_stats(cfg)
    mu = re.astype(np.float64) + 1j * im.astype(np.float64)
    absm = ab.astype(np.float64)
    G = cfg.group
    keys, spent = 0, 0.0
    for unit, g in pairs:
        n = int(u.lengths[unit])
        layer = int(u.unit_layer[unit])
        k_bits = synth.key_rows(cfg, unit, g)
        v_bits = synth.value_rows(cfg, unit, g)
        pos = synth.positions(cfg, unit)
        t0 = time.perf_counter()
        rows = o.bf16_bits_to_f64(k_bits)
        raw = np.stack([o.score_head(rows, pos, int(u.q_pos[unit]), mu[layer, h], absm[layer, h], cfg.head_dim,
                                     cfg.pairing, cfg.rope_base, cfg.offsets, form, cfg.offset_reduce)
                        for h in range(g * G, (g + 1) * G)])
        agg = o.aggregate_unit(raw, n, G, cfg.sink, cfg.window, cfg.agg)[0]
        kept = o.select(agg, int(u.budget[unit]))
        o.compact(k_bits, kept)
        o.compact(v_bits, kept)
        o.compact(pos, kept)
        spent += time.perf_counter() - t0
        keys += n
    return keys, spent, len(pairs)


def host_cores() -> int:
    """Host threads for the oracle pool: the cores this process may run on, at most 16
    (a one-GPU share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(cfg, seconds: float) -> dict:
    """The fp64 oracle as it stands, on every host core (one process per core), on a
    bounded sample of the same workload: whole (unit, KV head) pairs in order, as many
    per worker as one worker gets through in about `seconds` of oracle time (from a
    trial of one pair per worker, all workers at once).  Timed in both of its forms for the mean over offsets: the
    folded dot product (`value`) and the direct per-offset sum; the maximum over
    offsets has only the direct form.  A form's rate is all the keys over the slowest
    worker's oracle time."""
    import concurrent.futures as cf
    import multiprocessing as mp

    workers = host_cores()
    all_pairs = [(unit, g) for unit in range(cfg.n_units) for g in range(cfg.n_kv_heads)]
    forms = ["direct"] if cfg.offset_reduce == "max" else ["folded", "direct"]
    out = {}
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"),
                                initializer=_baseline_init) as ex:
        list(ex.map(_baseline_ready, range(workers)))
        for form in forms:
            # one pair per worker, all at once: the per-pair time under the same contention
            trial = list(ex.map(_baseline_pairs, [(cfg, [all_pairs[w % len(all_pairs)]], form)
                                                  for w in range(workers)]))
            t_pair = max(r[1] for r in trial)
            per = max(1, int(round(seconds / max(t_pair, 1e-3))))
            take = [all_pairs[i % len(all_pairs)] for i in range(workers * per)]
            jobs = [(cfg, take[w * per:(w + 1) * per], form) for w in range(workers)]
            res = list(ex.map(_baseline_pairs, jobs))
            keys = sum(r[0] for r in res)
            slow = max(r[1] for r in res)
            out[form] = {"value": keys / slow / 1e6, "pairs": sum(r[2] for r in res), "keys": keys,
                         "slowest_worker_s": slow}
    main_form = forms[0]
    desc = {"folded": "folded form", "direct": "direct form"}
    return {"value": out[main_form]["value"], "unit": "M keys/s", "cores": workers, "kind": "oracle",
            "sample": f"{out[main_form]['pairs']} (unit, KV head) pairs = {out[main_form]['keys']} keys of "
                      f"{cfg.name} ({per_note(out[main_form], workers)}), fp64 {desc[main_form]}"
                      f"{', maximum over offsets' if cfg.offset_reduce == 'max' else ''}, one process per core",
            "forms": {f: dict(v, unit="M keys/s") for f, v in out.items()},
            "host_cpus": os.cpu_count()}


def per_note(r: dict, workers: int) -> str:
    return f"{r['pairs'] // workers} per worker, slowest worker {r['slowest_worker_s']:.1f} s of oracle time"


def recorded_traffic(kernel: str, workload: str):
    """A kernel's HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if one exists and the kernel sources are the ones it measured;
    else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "#")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in ("tria_kernels.hip", "tria_kernels.h"):
        with open(os.path.join(ROOT, "key_importance_scoring_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if fields.get("kernel_sources_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def copy_probe(gb: float, steps: int) -> int:
    """A plain copy of a known number of bytes (torch's copy kernel): its time gives the
    achievable streaming bandwidth, and its FETCH_SIZE / WRITE_SIZE counters the factor
    that turns counter readings into bytes."""
    import torch
    n = int(gb * 1e9) // 16 * 16
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "ms": ms,
                      "GBps_read_plus_write": 2 * n / (ms / 1e3) / 1e9}))
    return 0


def read_probe(args) -> int:
    """The streaming-read probe (libtria_probe.so): `--read-probe` GB read once per step
    by a persistent grid of `--probe-wgs-per-cu` workgroups per compute unit in tiles of
    `--probe-tile-kib` KiB, the score kernel's access shape.  Its rate is the practical
    read ceiling the score kernel is compared with."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "key_importance_scoring_amd", "libtria_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run python -m key_importance_scoring_amd.build")
    lib = ctypes.CDLL(path)
    lib.tria_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.tria_probe_read.restype = ctypes.c_int
    n = int(args.read_probe * 1e9) // 16 * 16
    tile = args.probe_tile_kib * 1024
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = args.probe_wgs_per_cu * cus
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(0x5A)
    sink = torch.zeros(grid, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()

    def launch():
        rc = lib.tria_probe_read(src.data_ptr(), n, tile, grid, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"tria_probe_read failed: {rc}")

    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        launch()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    print(json.dumps({"probe": "read", "kernel": "k_read_probe", "bytes_read": n, "tile_bytes": tile, "grid": grid,
                      "compute_units": cus, "steps": args.steps, "ms": ms, "GBps_read": n / (ms / 1e3) / 1e9,
                      "frac_of_hbm_peak": n / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS}))
    return 0


CALIB_METRIC = "G pre-RoPE query rows reduced to calibration statistics/s; % of HBM peak GB/s"


def calib_cpu_baseline(cfg, T: int, seconds: float) -> dict:
    """oracle.calibrate as it stands on whole (layer, query head) streams, in order,
    until `seconds` of oracle time have passed."""
    from threadpoolctl import threadpool_limits
    from key_importance_scoring_amd import synth
    from oracle import tria_oracle as o

    rows = 0
    spent = 0.0
    heads = 0
    with threadpool_limits(1):
        for l in range(cfg.n_layers):
            for h in range(cfg.n_q_heads):
                q = synth.query_rows(cfg, l, h, T)
                t0 = time.perf_counter()
                o.calibrate(q, cfg.pairing)
                spent += time.perf_counter() - t0
                rows += T
                heads += 1
                if spent >= seconds:
                    break
            if spent >= seconds:
                break
    return {"value": rows / spent / 1e9, "unit": "G rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{heads} (layer, query head) streams of {T} rows of {cfg.name}, fp64, "
                      f"{spent:.1f} s on one host thread",
            "host_cpus": os.cpu_count()}


def bench_calibrate(args) -> int:
    """The calibration reduction: tria_calibrate over a [L][Hq][T][d] stream of
    pre-RoPE query rows resident in HBM."""
    import numpy as np
    import torch
    from key_importance_scoring_amd import _lib as L
    from key_importance_scoring_amd import synth
    from key_importance_scoring_amd.device import calibrate, params_for

    cfg = synth.CONFIGS[args.config]
    T = args.tokens
    print(f"[bench] building the {cfg.name} query stream, {T} tokens", file=sys.stderr, flush=True)
    q = None
    path = ""
    if args.input_cache:
        os.makedirs(args.input_cache, exist_ok=True)
        path = os.path.join(args.input_cache, f"{cfg.name}_s{cfg.seed}_q{T}.npy")
        if os.path.exists(path):
            q = np.load(path, mmap_mode="r")
    if q is None:
        q = synth.query_stream(cfg, T)
        if path:
            np.save(path, q)
    qd = torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).to("cuda:0")
    del q
    p = params_for(cfg)
    stream = torch.cuda.current_stream()
    print("[bench] warmup", file=sys.stderr, flush=True)
    out = calibrate(p, qd, stream=stream)        # also the copy the timed outputs must equal
    for _ in range(args.warmup - 1):
        calibrate(p, qd, stream=stream)
    torch.cuda.synchronize()
    # outputs and workspace allocated once; the timed region is the entry point alone
    F = cfg.head_dim // 2
    ws_bytes = L.tria_calibrate_workspace_size(p, T)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    o5 = [torch.empty((cfg.n_layers, cfg.n_q_heads, F), dtype=torch.float32, device="cuda:0") for _ in range(5)]

    def step():
        L.tria_calibrate(p, qd, qd.stride(0), qd.stride(1), qd.stride(2), T, *o5, ws, ws_bytes, stream)

    def region(kernel_events: bool):
        L.tria_timing_read()
        L.tria_timing_enable(kernel_events)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(args.steps):
            step()
        t1.record(stream)
        torch.cuda.synchronize()
        L.tria_timing_enable(False)
        return t0.elapsed_time(t1) / args.steps, L.tria_timing_read()

    ms, _ = region(False)
    ms_inst, kt = region(True)
    for a, b in zip(o5, (out["q_mean_re"], out["q_mean_im"], out["q_abs_mean"], out["r"], out["mrl"])):
        assert torch.equal(a, b)
    rows = cfg.n_layers * cfg.n_q_heads * T
    # algorithmic bytes: every query row read once, five fp32 statistics per band written
    alg = rows * cfg.head_dim * 2 + 5 * cfg.n_layers * cfg.n_q_heads * F * 4
    kms = kt["k_calib"][0] / kt["k_calib"][1]
    achieved = alg / (kms / 1e3) / 1e9
    print(f"[bench] {ms:.4f} ms/step ({ms_inst:.4f} with events), k_calib + k_calib_final {kms:.4f} ms",
          file=sys.stderr, flush=True)
    base = calib_cpu_baseline(cfg, T, args.cpu_seconds) if args.cpu_seconds > 0 else None
    print(json.dumps({
        "metric": CALIB_METRIC,
        "value": rows / (ms / 1e3) / 1e9,
        "unit": "G rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"calibrate_{cfg.name}", "layers": cfg.n_layers, "q_heads": cfg.n_q_heads,
                   "head_dim": cfg.head_dim, "tokens": T, "pairing": cfg.pairing},
        "hbm_algorithmic_GBps": alg / (ms / 1e3) / 1e9,
        "hbm_pct_of_peak": 100.0 * alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
        "algorithmic_bytes_per_step": alg,
        "kernel_ms": {"k_calib+k_calib_final": kms},
        "roofline": {"kernel": "k_calib (with k_calib_final)", "bound": "hbm", "achieved": achieved,
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic("k_calib", f"calibrate_{cfg.name}"),
                     "algorithmic_bytes_per_launch": alg},
        "cpu_baseline": base,
    }))
    return 0


DECODE_METRIC = "M keys scored+selected+compacted/s in a decode loop (prune every 128 tokens); % of HBM peak GB/s"


def bench_decode(args) -> int:
    """The decode loop: 64 sequences x 8 KV heads (d 128, G 4, NEOX) hold a budget of
    2048 slots; every step appends 128 tokens to each and prunes them back in place
    (score -> select -> in-place compaction), the port's regime (interval 128, window
    256, sink 0).  A step's new rows are resident in HBM before the timed region."""
    import numpy as np
    import torch
    from key_importance_scoring_amd import _lib as L
    from key_importance_scoring_amd import synth
    from key_importance_scoring_amd.decode import DecodeLoop

    cfg = synth.CONFIGS["batched_decode"].replace(name="decode_loop", n_seqs=64, ragged_min=0, window=256, sink=0,
                                                  offset_reduce=args.offsets)
    budget, interval = 2048, 128
    loop = DecodeLoop(cfg, budget, interval)
    n_fill = -(-budget // interval)                      # appends until the first prune
    n_steps = n_fill + args.warmup + 2 * args.steps     # the fill, warm-up and both timed regions
    print(f"[bench] decode loop: generating {n_steps} steps of rows", file=sys.stderr, flush=True)
    rows = [loop.upload(*loop.new_rows(interval, p0=i * interval)) for i in range(n_steps)]
    for i in range(n_fill):
        loop.step(rows=rows[i])
    for i in range(n_fill, n_fill + args.warmup):
        loop.step(rows=rows[i])
    torch.cuda.synchronize()
    assert loop.prunes >= 1

    stream = torch.cuda.current_stream()

    def region(kernel_events: bool, first: int):
        L.tria_timing_read()
        L.tria_timing_enable(kernel_events)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for i in range(first, first + args.steps):
            assert loop.step(rows=rows[i], stream=stream)
        t1.record(stream)
        torch.cuda.synchronize()
        L.tria_timing_enable(False)
        return t0.elapsed_time(t1) / args.steps, L.tria_timing_read()

    ms, _ = region(False, n_fill + args.warmup)
    ms_inst, kt = region(True, n_fill + args.warmup + args.steps)
    assert loop.flags() == 0
    per_kernel = {k: v[0] / v[1] for k, v in kt.items() if v[1]}
    U, Hkv, d = cfg.n_units, cfg.n_kv_heads, cfg.head_dim
    n = budget + interval
    keys = U * Hkv * n                                   # head-keys scored per prune
    score_bytes = keys * 2 * d
    # compaction: every kept row that moves is read and written (K and V) with its
    # position; at most all of them
    cmp_bytes = U * Hkv * budget * (4 * 2 * d + 8)
    alg = score_bytes + cmp_bytes + U * Hkv * interval * (4 * d + 4)   # + the appended rows
    # the dominant kernel is the in-place compaction (its timing id is k_compact):
    # nearly every kept row moves when the evicted slots are spread out
    cmp_ms = per_kernel["k_compact"]
    achieved = cmp_bytes / (cmp_ms / 1e3) / 1e9
    print(f"[bench] {ms:.4f} ms/step ({ms_inst:.4f} with events), kernels {per_kernel}", file=sys.stderr, flush=True)
    print(json.dumps({
        "metric": DECODE_METRIC,
        "value": keys / (ms / 1e3) / 1e6,
        "unit": "M keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_loop", "sequences": U, "kv_heads": Hkv, "q_heads": cfg.n_q_heads,
                   "head_dim": d, "budget": budget, "interval": interval, "window": cfg.window, "sink": cfg.sink,
                   "paged": True, "block_size": cfg.block_size, "offset_reduce": cfg.offset_reduce,
                   "step": "append 128 tokens per sequence + prune in place"},
        "prune_overhead_us_per_generated_token": ms * 1e3 / interval,
        "hbm_algorithmic_GBps_upper_bound": alg / (ms / 1e3) / 1e9,
        "algorithmic_bytes_per_step_upper_bound": alg,
        "kernel_ms": per_kernel,
        "roofline": {"kernel": "k_compact_inplace", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic("k_compact_inplace", "decode_loop"),
                     "algorithmic_bytes_per_launch": cmp_bytes,
                     "algorithmic_bytes_note": "every kept row's K and V read and written with its position (an "
                                               "upper bound: rows whose slot does not change are not moved)",
                     "score_kernel_GBps": score_bytes / (per_kernel["k_score"] / 1e3) / 1e9},
        "cpu_baseline": None,
    }))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; 200 with --calibrate, 20 with --decode-loop)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="warmup steps (default 100; 50 with --calibrate, 10 with --decode-loop)")
    ap.add_argument("--config", default="qwen3_8b")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget (0: skip)")
    ap.add_argument("--input-cache", default="", metavar="DIR",
                    help="keep the generated K/V caches as .npy files in DIR and reuse them")
    ap.add_argument("--copy-probe", type=float, default=0.0, metavar="GB",
                    help="instead of the pass, time a plain device-to-device copy of GB gigabytes "
                         "(the reference kernel for scaling HBM byte counters)")
    ap.add_argument("--read-probe", type=float, default=0.0, metavar="GB",
                    help="instead of the pass, time the streaming-read probe over GB gigabytes (2.415919104: "
                         "the Qwen3-8B-shaped K cache)")
    ap.add_argument("--probe-tile-kib", type=int, default=512, help="read probe tile (KiB; default 512)")
    ap.add_argument("--probe-wgs-per-cu", type=int, default=2, help="read probe workgroups per compute unit")
    ap.add_argument("--no-extra", dest="extra", action="store_false",
                    help="time only --config (the default Qwen3-8B line also times the Qwen3-32B-shaped pass)")
    ap.add_argument("--calibrate", action="store_true",
                    help="instead of the pass, time the calibration reduction (tria_calibrate) over a "
                         "synthetic pre-RoPE query stream of --tokens rows per (layer, query head)")
    ap.add_argument("--tokens", type=int, default=8192, help="calibration tokens (with --calibrate)")
    ap.add_argument("--decode-loop", action="store_true",
                    help="instead of the single pass, time the decode loop (append 128 tokens, prune in place)")
    ap.add_argument("--offsets", choices=("mean", "max"), default="mean",
                    help="reduction over the future offsets: the mean (the method) or the maximum variant")
    ap.add_argument("--select", choices=("auto", "per_group", "tiled"), default="auto",
                    help="tria_select's work distribution (auto: the library's default)")
    args = ap.parse_args()
    # The clocks ramp for tens of milliseconds after the host's set-up: a pass needs ~30
    # warm-up steps to reach its steady rate (3 left the Qwen3-8B-shaped pass ~3 % slow).
    # A calibration step is ~0.4 ms: more of them keep the timed region near 0.1 s.  The
    # decode loop generates every step's rows on the host, so it runs fewer.
    if args.steps is None:
        args.steps = 200 if args.calibrate else (20 if args.decode_loop else 50)
    if args.warmup is None:
        args.warmup = 50 if args.calibrate else (10 if args.decode_loop else 100)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the pass shards with no "
              f"exchange, so N GPUs run N independent copies of this measurement)", file=sys.stderr)
        return 2

    import torch
    if args.copy_probe > 0:
        return copy_probe(args.copy_probe, args.steps)
    if args.read_probe > 0:
        return read_probe(args)
    if args.calibrate:
        return bench_calibrate(args)
    if args.decode_loop:
        return bench_decode(args)
    from key_importance_scoring_amd import _lib as L
    from key_importance_scoring_amd import synth

    L.tria_select_strategy({"auto": L.SELECT_AUTO, "per_group": L.SELECT_PER_GROUP,
                            "tiled": L.SELECT_TILED}[args.select])
    cfg = synth.CONFIGS[args.config]
    if args.offsets == "max":
        cfg = cfg.replace(name=f"{cfg.name}_offsets_max", offset_reduce="max")
    r = time_pass(cfg, args)
    extra = {}
    # the default line also carries the Qwen3-32B-shaped pass (same steps and warmup)
    if args.extra and args.config == "qwen3_8b" and args.offsets == "mean":
        for name in ("qwen3_32b",):
            e = time_pass(synth.CONFIGS[name], args)
            extra[name] = {"value": e["value"], "unit": "M keys/s", "ms_per_step": e["ms"],
                           "hbm_algorithmic_GBps": e["alg_GBps"], "hbm_pct_of_peak": e["pct"],
                           "algorithmic_bytes_per_step": e["alg"], "head_keys_per_step": e["keys"],
                           "kernel_ms": e["per_kernel"], "roofline": e["roofline"],
                           "config": workload_desc(synth.CONFIGS[name])}

    base = None
    if args.cpu_seconds > 0:
        print(f"[bench] oracle CPU baseline ({host_cores()} processes)", file=sys.stderr, flush=True)
        base = cpu_baseline(cfg, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": r["value"],
        "unit": "M keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(workload_desc(cfg), **({"select": args.select} if args.select != "auto" else {})),
        "hbm_algorithmic_GBps": r["alg_GBps"],
        "hbm_pct_of_peak": r["pct"],
        "algorithmic_bytes_per_step": r["alg"],
        "head_keys_per_step": r["keys"],
        "kernel_ms": r["per_kernel"],
        "kernel_timing": {"source": "HIP events on the launch stream around each library launch, over a second "
                                    "region of the same K steps after the timed one",
                          "ms_per_step_with_kernel_events": r["ms_inst"]},
        "roofline": r["roofline"],
        "cpu_baseline": base,
    }
    if extra:
        out["extra_workloads"] = extra
    print(json.dumps(out))
    return 0


def time_pass(cfg, args) -> dict:
    """Builds cfg's inputs on the device, runs W warmup steps, then times K steps twice:
    once bare (the measurement) and once with HIP events around every library launch
    (per-kernel times).  The device buffers are released before it returns."""
    import torch
    from key_importance_scoring_amd import _lib as L
    from key_importance_scoring_amd.device import DeviceProblem

    cache_name = cfg.name.replace("_offsets_max", "")   # the offset reduction does not change the inputs
    print(f"[bench] building {cfg.name} inputs", file=sys.stderr, flush=True)
    hosts = {}
    if args.input_cache:
        import numpy as np
        from key_importance_scoring_amd.device import host_cache
        os.makedirs(args.input_cache, exist_ok=True)
        for which in ("k", "v"):
            path = os.path.join(args.input_cache, f"{cache_name}_s{cfg.seed}_{which}.npy")
            if os.path.exists(path):
                hosts[which] = np.load(path, mmap_mode="r")
            else:
                hosts[which] = host_cache(cfg, which)
                np.save(path, hosts[which])
    # the pass as a serving engine runs it: aggregates only, no per-query-head scores
    prob = DeviceProblem(cfg, device="cuda:0", keep_raw=False, k_host=hosts.get("k"), v_host=hosts.get("v"))
    hosts.clear()
    stream = torch.cuda.current_stream()
    print(f"[bench] {cfg.name} warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        prob.run(stream)
    torch.cuda.synchronize()

    def region(kernel_events: bool):
        """K steps bracketed by a synchronize and HIP events on the launch stream; with
        kernel_events the library also brackets each of its launches with HIP events."""
        L.tria_timing_read()
        L.tria_timing_enable(kernel_events)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record(stream)
        for _ in range(args.steps):
            prob.run(stream)
        t1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        L.tria_timing_enable(False)
        kt = L.tria_timing_read()
        return t0.elapsed_time(t1) / args.steps, wall, kt

    # the timed region: K steps with no per-kernel events (each recorded event idles
    # the GPU for several microseconds between kernels)
    ms, wall, _ = region(False)
    # then K more steps with every kernel bracketed by HIP events, for per-kernel times
    ms_inst, _, kt = region(True)
    assert prob.flags() == 0

    keys = prob.head_keys()
    alg = prob.algorithmic_bytes()
    per_kernel = {k: v[0] / v[1] for k, v in kt.items() if v[1]}
    dom = max(per_kernel, key=per_kernel.get)
    # algorithmic bytes of k_score per launch: every cached K row read once
    score_bytes = keys * 2 * cfg.head_dim
    # its useful MFMA work: per (key, query head) a d-long dot product per offset
    # (maximum variant) or one folded dot product (the mean), plus the norm term's d/2
    dots = len(cfg.offsets) if cfg.offset_reduce == "max" else 1
    score_kernel = "k_score_max" if cfg.offset_reduce == "max" else "k_score"
    score_flops = keys * cfg.group * 2 * (cfg.head_dim * dots + cfg.head_dim // 2)
    score_ms = per_kernel["k_score"]
    achieved = score_bytes / (score_ms / 1e3) / 1e9
    print(f"[bench] {cfg.name}: {ms:.3f} ms/step ({ms_inst:.3f} with per-kernel events), wall "
          f"{wall / args.steps * 1e3:.3f} ms/step, kernels {per_kernel}", file=sys.stderr, flush=True)
    del prob
    torch.cuda.empty_cache()
    return {
        "ms": ms, "ms_inst": ms_inst, "keys": keys, "alg": alg, "per_kernel": per_kernel,
        "value": keys / (ms / 1e3) / 1e6,
        "alg_GBps": alg / (ms / 1e3) / 1e9,
        "pct": 100.0 * alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
        "roofline": {"kernel": score_kernel, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "traffic": recorded_traffic(score_kernel, cfg.name),
                     "algorithmic_bytes_per_launch": score_bytes, "dominant_kernel": dom,
                     "mfma_bf16_tflops": score_flops / (score_ms / 1e3) / 1e12,
                     "mfma_frac_of_bf16_dense_peak": score_flops / (score_ms / 1e3) / 2.5e15},
    }


if __name__ == "__main__":
    sys.exit(main())
