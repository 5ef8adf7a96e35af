"""Decode hot-path benchmark on one MI355X.

One step = one decode layer-step of the whole batch: quantise-append of the
new entry and indexer key, lightning-indexer scan + causal mask + top-k (the
append carried in the scan's launch), and sparse absorbed-MLA decode (+ window
branch).  The CSA2 group configuration
counts one group (Full + Reindex + 4 Reuse layers) as a step.

Default workload: the V3.2-shaped long-context configuration (B = 4,
T = 131072, E4M3 caches with 656-byte main rows and 132-byte indexer rows,
128 heads, 64 x 128 indexer, top-2048).  Inputs are seeded synthetic N(0, 1)
tensors; caches are built by the library's own append.  Eight distinct layer
caches are rotated so that the working set is far larger than the on-chip
caches.

Prints ONE JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import contextlib
import gc
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode layer-steps/s at T=128K; achieved HBM GB/s vs roofline"
HBM_PEAK_GBPS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default="c3", choices=["c1", "c2", "c3", "c4", "c4x", "c5"])
    p.add_argument("--layers", type=int, default=8, help="distinct layer caches rotated")
    p.add_argument("--pool", type=int, default=0,
                   help="CSA2 group: the Full layer publishes a candidate pool of this many 8-position "
                        "blocks and the Reindex layer scores only the pool (hierarchical sparse indexer)")
    p.add_argument("--win-fmt", default="bf16", choices=["bf16", "mxfp8"],
                   help="window entries as bf16 or as MXFP8 (V4.1's 528-byte entry at 512 channels)")
    p.add_argument("--compress", type=int, default=0, metavar="M",
                   help="pool the step's main entry from M tokens with the CSA2 compressor (mla_compress_append)")
    p.add_argument("--queries", type=int, default=0, metavar="G",
                   help="G positions of one sequence per step (a prefill chunk / multi-token prediction): "
                        "the step appends G entries, then one indexer call and one decode call serve the G "
                        "queries over the shared cache (each with its own causal limit)")
    p.add_argument("--score-bf16", action="store_true",
                   help="the bf16-score top-k: index scores rounded to bf16 before they are selected")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-side-configs", action="store_true",
                   help="skip the short runs of c2, c4, c4x and c5 that the default c3 invocation reports")
    p.add_argument("--graph", action="store_true",
                   help="replay each rotated layer's step from a HIP graph captured once (the stamped steps "
                        "still run eagerly); default: every step's kernels are launched from the host")
    p.add_argument("--python-group", action="store_true",
                   help="enqueue each step through csa2_group_step (one Python call per layer and kernel) "
                        "instead of mla_csa2_group_step (one C call per step)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="time only torch's device copy of a known size (scales HBM byte counters)")
    return p.parse_args()


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


class Layer:
    """Caches and per-layer inputs of one rotated layer (or one CSA2 group)."""


def build_layers(cfg, n_layers, seed=0):
    import numpy as np
    import torch

    import sparse_latent_attention_mla_amd as M
    import workloads as WL

    dev = "cuda"
    B, N, D, H = cfg.B, cfg.N, cfg.D, cfg.H
    mr = M.Row(cfg.main_fmt, cfg.dim, cfg.rope)
    ir = M.Row(cfg.idx_fmt, cfg.d_I, 0)
    qdt = torch.float32 if cfg.main_fmt == WL.F32 else torch.bfloat16
    L_grp = len(cfg.layers)
    n_idx = WL.n_indexers(cfg)
    layers = []
    for l in range(n_layers):
        t0 = time.time()
        off = 16 * l                      # tensor-id offset of rotated layer l (layer 0 = the standard inputs)
        X = Layer()
        X.main = torch.empty((B, N, M.row_bytes(mr)), dtype=torch.uint8, device=dev)
        X.idx = torch.empty((B, N, M.row_bytes(ir)), dtype=torch.uint8, device=dev)
        slots_all = torch.arange(N, dtype=torch.int32, device=dev).expand(B, N).contiguous()
        if cfg.m == 1:
            chunk = max(1, (1 << 26) // (N * D))      # sequences per generation chunk
            for b0 in range(0, B, chunk):
                b1 = min(B, b0 + chunk)
                # positions of sequences b0..b1 in the [B, N, D] streams
                main = WL.normal(seed, cfg.cid, WL.T_MAIN + off, (b1 - b0, N, D), offset=b0 * N * D)
                idx = WL.normal(seed, cfg.cid, WL.T_IDX + off, (b1 - b0, N, cfg.d_I), offset=b0 * N * cfg.d_I)
                M.mla_kv_append_quant(mr, ir, torch.from_numpy(main).to(dev), torch.from_numpy(idx).to(dev),
                                      slots_all[b0:b1].contiguous(), X.main[b0:b1], X.idx[b0:b1])
                del main, idx
        else:
            # m tokens per entry: each entry pooled by the CSA2 compressor on the GPU (unit norm
            # weight, no rotation) straight into its row; the indexer key appended on its own
            slot0 = torch.zeros(N, dtype=torch.int32, device=dev)    # each entry is its own one-row "sequence"
            ce = 1 << 15
            for b in range(B):
                for n0 in range(0, N, ce):
                    n1 = min(N, n0 + ce)
                    kv, gate = WL.compressor_tokens(cfg, seed, b, n0, n1, tensor_offset=off)
                    M.mla_compress_append(mr, torch.from_numpy(kv).to(dev), torch.from_numpy(gate).to(dev),
                                          X.main[b, n0:n1].unsqueeze(1), slot0[:n1 - n0], None, 1e-6)
                    del kv, gate
                idx = WL.normal(seed, cfg.cid, WL.T_IDX + off, (1, N, cfg.d_I), offset=b * N * cfg.d_I)
                M.mla_kv_append_quant(mr, ir, None, torch.from_numpy(idx).to(dev), slots_all[b:b + 1].contiguous(),
                                      None, X.idx[b:b + 1])
                del idx
        # the entry appended by each step (position N-1), and the step's queries
        X.new_main = torch.from_numpy(WL.normal(seed, cfg.cid, 100 + off, (B, 1, D))).to(dev)
        X.new_idx = torch.from_numpy(WL.normal(seed, cfg.cid, 101 + off, (B, 1, cfg.d_I))).to(dev)
        q = WL.normal(seed, cfg.cid, WL.T_Q + off, (L_grp, B, H, D))
        qi = WL.normal(seed, cfg.cid, WL.T_QIDX + off, (n_idx, B, cfg.H_I, cfg.d_I))
        X.q = torch.from_numpy(q).to(dev).to(qdt)
        X.q_idx = torch.from_numpy(qi).to(dev).to(qdt)
        X.w = torch.from_numpy(WL.normal(seed, cfg.cid, WL.T_W + off, (n_idx, B, cfg.H_I)) *
                               np.float32(cfg.w_scale)).to(dev)
        if cfg.W:
            X.win = torch.from_numpy(WL.normal(seed, cfg.cid, WL.T_WIN + off, (L_grp, B, cfg.W, D))).to(dev).to(
                torch.bfloat16).contiguous()
            X.new_win = torch.from_numpy(WL.normal(seed, cfg.cid, 102 + off, (L_grp, B, D))).to(dev)
        torch.cuda.synchronize()
        layers.append(X)
        log(f"layer {l} built in {time.time() - t0:.1f}s")
    return layers


SCAN_SOURCES = ("csrc/indexer.hip", "csrc/append.hpp", "csrc/common.hpp", "csrc/launch.hpp", "build.py")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_scan_c3_hbm_traffic.md")


PACE_EVERY, PACE_AHEAD = 8, 16


@contextlib.contextmanager
def gc_paused():
    """Python's cyclic garbage collector paused (after one full collection): a collection
    of the whole heap takes tens of ms, during which a host that keeps the GPU only a few
    steps ahead leaves it idle (a serving loop runs the same way)."""
    gc.collect()
    gc.disable()
    try:
        yield
    finally:
        gc.enable()


def paced_loop(run_step, steps, stream):
    """run_step(i) for i < steps, the host at most PACE_AHEAD + PACE_EVERY steps ahead of
    the GPU (an event every PACE_EVERY steps; before recording one, the host waits for the
    one recorded that many steps earlier). The GPU stays fed; without the bound, a host that enqueues faster than the GPU
    runs piles up thousands of launches, and the runtime then stalls while it recycles
    their resources, leaving the GPU idle between kernels (a c5 group: 288 instead of
    130 us on some runs)."""
    import torch
    marks = [torch.cuda.Event() for _ in range(PACE_AHEAD // PACE_EVERY + 1)]
    for i in range(steps):
        if i % PACE_EVERY == 0:
            m = (i // PACE_EVERY) % len(marks)
            if i >= PACE_AHEAD + PACE_EVERY:
                marks[m].synchronize()                 # recorded PACE_AHEAD + PACE_EVERY steps ago
            marks[m].record(stream)
        run_step(i)


def scan_source_digest():
    """sha256 over the sources the indexer scan kernel is compiled from."""
    h = hashlib.sha256()
    for f in SCAN_SOURCES:
        with open(os.path.join(ROOT, "sparse_latent_attention_mla_amd", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def scan_traffic(cfg):
    """HBM bytes per scan launch from the committed counter summary: FETCH_SIZE +
    WRITE_SIZE per dispatch, each scaled by what the counter reads for a plain copy
    of known size.  None when the summary is absent, is for another workload, or
    was taken from a different version of the kernel's sources."""
    if cfg.name != "c3" or not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            if line.startswith("    ") and "=" in line:
                key, val = line.strip().split("=", 1)
                kv[key.strip()] = val.strip()
    try:
        if kv["scan_source_sha256"] != scan_source_digest():
            return None
        fetch = float(kv["scan_fetch_kib"]) * 1024 * float(kv["fetch_factor"])
        write = float(kv["scan_write_kib"]) * 1024 * float(kv["write_factor"])
    except (KeyError, ValueError):
        return None
    return fetch + write


def calibrate_copy(args):
    """Copies of a known size, for scaling the HBM byte counters: each launch must
    read and write exactly COPY_BYTES.  Two kernels: the runtime's device-to-device
    copy (what torch's copy_ issues) and torch's elementwise negation into another
    buffer, a copy-shaped kernel of the ordinary kind."""
    import torch
    torch.cuda.set_device(0)
    n = COPY_BYTES // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    res = {"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES}
    for name, fn in (("copy_", lambda: dst.copy_(src)), ("neg", lambda: torch.neg(src, out=dst))):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1e3 / args.steps
        res[name] = {"avg_us": us, "gbps_read_plus_write": 2 * COPY_BYTES / (us * 1e-6) / 1e9}
    print(json.dumps(res), flush=True)


COPY_BYTES = 1 << 30


SIDE_CONFIGS = ("c2", "c4", "c4x", "c5")      # reported beside the headline in the same run


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the decode path runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args)
        return
    import torch

    import workloads as WL

    cfg = WL.CONFIGS[args.config]
    if args.queries:
        return multi_query(args, cfg)
    torch.cuda.set_device(0)
    head = run_config(args, cfg, max(1, args.layers), args.steps, args.warmup, headline=True)
    result = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "launch": head["launch"],
        "ms_per_step_eager": head["ms_per_step_eager"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "step_roofline": head["step_roofline"],
        "per_kernel_breakdown": head["per_kernel_breakdown"],
    }
    if "csa2_flushed" in head:
        result["csa2_flushed"] = head["csa2_flushed"]
    # the other configurations, shortly, in the same run (default invocation only)
    if args.config == "c3" and not (args.pool or args.compress or args.graph or args.score_bf16 or
                                    args.win_fmt != "bf16" or args.no_side_configs):
        side = {}
        for name in SIDE_CONFIGS:
            torch.cuda.empty_cache()
            r = run_config(args, WL.CONFIGS[name], 4, max(20, min(args.steps, 200)), max(5, min(args.warmup, 20)),
                           headline=False)
            side[name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "launch")}
            side[name]["step_frac"] = r["step_roofline"]["frac"]
            side[name]["scan_frac"] = r["roofline"]["frac"]
            side[name]["scan_avg_launch_us"] = r["roofline"]["avg_launch_us"]
            side[name]["per_kernel_breakdown"] = r["per_kernel_breakdown"]
            if "csa2_flushed" in r:
                side[name]["csa2_flushed"] = r["csa2_flushed"]
            log(f"{name}: {r['ms_per_step'] * 1e3:.2f} us/step, step {100 * side[name]['step_frac']:.1f} % of "
                f"8 TB/s, scan {100 * side[name]['scan_frac']:.1f} %")
        result["configs"] = side
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(result), flush=True)


def run_config(args, cfg, n_layers, steps, warmup, headline):
    """Build rotated layer caches for cfg, time `steps` steps (the group helper's calls),
    then the roofline pass (every indexer scan stamped, outside the timed steps) and the
    per-kernel breakdown pass. Returns the figures."""
    import numpy as np
    import torch

    import sparse_latent_attention_mla_amd as M
    import workloads as WL

    dev = "cuda"
    B, N, H = cfg.B, cfg.N, cfg.H
    mr = M.Row(cfg.main_fmt, cfg.dim, cfg.rope)
    ir = M.Row(cfg.idx_fmt, cfg.d_I, 0)
    L_grp = len(cfg.layers)
    log(f"config {cfg.name}: {cfg.desc}; building {n_layers} layer caches")
    layers = build_layers(cfg, n_layers)
    opt = args if headline else argparse.Namespace(pool=0, compress=0, win_fmt="bf16", graph=False,
                                                   score_bf16=False, python_group=False)
    win_fmt = M.MXFP8 if (cfg.W and opt.win_fmt == "mxfp8") else M.BF16
    if opt.compress:                                       # the window's projected kv and gate vectors
        for i, X in enumerate(layers):
            X.comp_kv = torch.from_numpy(WL.normal(0, cfg.cid, 200 + 2 * i, (B, opt.compress, cfg.D))).to(dev)
            X.comp_gate = torch.from_numpy(WL.normal(0, cfg.cid, 201 + 2 * i, (B, opt.compress, cfg.D))).to(dev)
        comp_norm = torch.ones(cfg.D, dtype=torch.float32, device=dev)
    if win_fmt == M.MXFP8:                                 # the same window values as MXFP8 entries
        for X in layers:
            ring8 = torch.zeros((X.win.shape[0], B, cfg.W, cfg.D + cfg.D // 32), dtype=torch.uint8, device=dev)
            for l in range(X.win.shape[0]):
                for s_ in range(cfg.W):
                    M.mla_kv_append_quant(mr, ir, None, None, None, None, None, X.win[l, :, s_].float().contiguous(),
                                          torch.full((B,), s_, dtype=torch.int32, device=dev), ring8[l])
            X.win = ring8
        torch.cuda.synchronize()

    k = cfg.k
    nvis = torch.full((B,), N, dtype=torch.int32, device=dev)
    slots = torch.full((B, 1), N - 1, dtype=torch.int32, device=dev)
    p_ = cfg.tokens - 1
    win_pos = torch.full((B,), p_, dtype=torch.int32, device=dev)
    win_len = torch.full((B,), min(cfg.W, p_ + 1), dtype=torch.int32, device=dev)
    idx_out = [torch.empty((B, k), dtype=torch.int32, device=dev) for _ in range(2)]
    out = torch.empty((L_grp, B, H, cfg.d_v), dtype=torch.float32, device=dev)
    lse = torch.empty((L_grp, B, H), dtype=torch.float32, device=dev)
    pool = opt.pool if WL.n_indexers(cfg) > 1 else 0
    POOL_BLOCK = 8
    ws_size = M.mla_indexer_topk_workspace(B, N, k)
    pool_args = None
    if pool:
        ws_size = max(ws_size, M.mla_indexer_pool_workspace(B, N, POOL_BLOCK))
        pool_args = (pool, POOL_BLOCK, torch.empty((B, N), dtype=torch.float32, device=dev),
                     torch.empty((B, pool * POOL_BLOCK), dtype=torch.int32, device=dev))
    ws_topk = torch.zeros(ws_size, dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(max(1, M.mla_sparse_decode_workspace(mr, cfg.d_v, B, H, k, cfg.W, win_fmt)), dtype=torch.uint8,
                         device=dev)
    stream = torch.cuda.current_stream()
    slots1 = slots[:, 0].contiguous()

    def step(X, between=None):
        """One layer-step (or CSA2 group) on layer caches X, as one mla_csa2_group_step call
        (or, with --python-group or a hook between layers, through csa2_group_step): the
        first layer appends the step's entry in its scan's launch (with --compress the main
        entry is pooled by mla_compress_append first), every layer its window entry."""
        if opt.compress:
            M.mla_compress_append(mr, X.comp_kv, X.comp_gate, X.main, slots1, comp_norm, 1e-6)
        kw = dict(new_main=None if opt.compress else X.new_main, new_idx=X.new_idx, slots=slots,
                  win_rings=X.win if cfg.W else None, new_win=X.new_win if cfg.W else None,
                  win_pos=win_pos if cfg.W else None, win_len=win_len if cfg.W else None,
                  pool=pool_args, score_bf16=opt.score_bf16)
        if between is not None or opt.python_group:
            M.csa2_group_step(mr, ir, cfg.layers, X.main, X.idx, nvis, k, cfg.sigma, cfg.softmax_scale, X.q,
                              X.q_idx, X.w, out, lse, ws_topk, ws_dec, idx_out, between_layers=between, **kw)
        else:                                              # the whole step in one C call
            M.mla_csa2_group_step(mr, ir, cfg.layers, X.main, X.idx, nvis, k, cfg.sigma, cfg.softmax_scale, X.q,
                                  X.q_idx, X.w, out, lse, ws_topk, ws_dec, idx_out, **kw)

    log(f"warmup {warmup} steps")
    for i in range(warmup):
        step(layers[i % n_layers])
    torch.cuda.synchronize()

    # one HIP graph per rotated layer cache, captured from the same calls (the
    # library only enqueues kernels: no allocation, no memset, no host sync)
    graphs = None
    if opt.graph:
        graphs = []
        for l in range(n_layers):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(layers[l])
            graphs.append(g)
        torch.cuda.synchronize()
        # replays must reproduce the eager step, also with eager work between them
        for rep_i in range(2):
            step(layers[1 % n_layers])
            torch.cuda.synchronize()
            ref = (out.clone(), lse.clone(), [x.clone() for x in idx_out])
            step(layers[0])
            graphs[1 % n_layers].replay()
            torch.cuda.synchronize()
            same_idx = all(torch.equal(torch.sort(a, dim=1)[0], torch.sort(b, dim=1)[0])
                           for a, b in zip(idx_out, ref[2]))
            # (the order of the selected positions may differ, and with it the
            # decode's summation order: outputs agree to rounding)
            close = lambda a, r: float((a - r).abs().max()) <= 1e-4 * float(r.abs().max())
            if not (same_idx and close(out, ref[0]) and close(lse, ref[1])):
                raise RuntimeError("graph replay differs from the eager step")
        log(f"captured {n_layers} step graphs; replays match the eager step")

    def run_step(i):
        if graphs is None:
            step(layers[i % n_layers])
        else:
            graphs[i % n_layers].replay()

    # timed region: exactly `steps` steps, nothing stamped
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with gc_paused():
        t_start.record(stream)
        paced_loop(run_step, steps, stream)
        t_end.record(stream)
        torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / steps

    # the same steps all launched from the host, for comparison (not the result)
    eager_ms = None
    if graphs is not None:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with gc_paused():
            e0.record(stream)
            paced_loop(lambda i: step(layers[i % n_layers]), steps, stream)
            e1.record(stream)
            torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / steps

    # roofline pass (outside the timed steps): whole eager steps with every indexer scan
    # stamped from its own dispatch: 96 steps, at least two per rotated cache, so that the
    # first launches after the idle gap do not weigh on the average
    for name in M.PROFILE_KERNELS:
        M.mla_profile_read(name)          # discard anything recorded before
    n_roof = max(96, 2 * n_layers)
    M.mla_profile_enable(("indexer_scan",))
    for i in range(n_roof):
        step(layers[i % n_layers])
    torch.cuda.synchronize()
    M.mla_profile_enable(())
    n_scan, scan_ms = M.mla_profile_read("indexer_scan")
    scan_us = scan_ms * 1e3 / n_scan

    # per-kernel breakdown: a separate pass with every kernel stamped
    n_brk = min(steps, 100)
    M.mla_profile_enable(M.PROFILE_KERNELS)
    for i in range(n_brk):
        step(layers[i % n_layers])
    torch.cuda.synchronize()
    M.mla_profile_enable(())
    per_kernel = {}
    for name in M.PROFILE_KERNELS:
        n, ms = M.mla_profile_read(name)
        if n:
            per_kernel[name] = {"launches": n, "avg_us": ms * 1e3 / n}

    res = {}
    if L_grp > 1:
        # the CSA2 group with a 512 MB scratch write between its layers (outside the timed
        # events; MoE layers intervene in the model): each layer timed on its own, the
        # Reindex layer no longer finding the keys the Full layer pulled through the caches
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(L_grp)]
        per_layer = np.zeros(L_grp)
        n_fl = min(steps, 20)
        for i in range(n_fl):
            def between(l):
                ev[l - 1][1].record(stream)
                scratch.fill_(l)
                ev[l][0].record(stream)
            scratch.fill_(0)
            ev[0][0].record(stream)
            step(layers[i % n_layers], between=between)
            ev[L_grp - 1][1].record(stream)
            torch.cuda.synchronize()
            per_layer += [ev[l][0].elapsed_time(ev[l][1]) for l in range(L_grp)]
        per_layer /= n_fl
        res["csa2_flushed"] = {
            "ms_per_group": float(per_layer.sum()),
            "ms_per_layer": {f"{l}:{m}": float(per_layer[l]) for l, m in enumerate(cfg.layers)},
            "groups": n_fl,
            "note": "eager launches, a 512 MB scratch write between layers outside the timed events; "
                    "value / ms_per_step are the back-to-back group",
        }
    log(f"{ms_per_step * 1e3:.2f} us/step" + (f" (eager {eager_ms * 1e3:.2f})" if eager_ms else "") +
        f"; scan {scan_us:.2f} us ({n_scan} stamped launches); breakdown pass (avg us): " +
        ", ".join(f"{kk}={v['avg_us']:.2f}" for kk, v in per_kernel.items()))

    ab = WL.algorithmic_bytes(cfg, pool, win_fmt=win_fmt)
    if opt.compress:                                       # m tokens' kv and gate in place of one fp32 entry
        ab["compress"] = B * opt.compress * cfg.D * 8 + cfg.D * 4 - B * cfg.D * 4
        ab["total"] += ab["compress"]
    step_gbps = ab["total"] / (ms_per_step * 1e-3) / 1e9
    # dominant kernel: the indexer scan (the first layer's carries the step's append).
    # Per launch it must read every visible indexer row of the batch plus the indexer
    # queries and head weights; the carried append's inputs and rows (entry and window)
    # are averaged over the group's scans; the scores it writes for the selection are
    # implementation traffic, not counted.
    n_idx_layers = WL.n_indexers(cfg)
    carried = B * (M.row_bytes(mr) + M.row_bytes(ir) + 4 * (cfg.D + cfg.d_I)) + (
        B * (4 * cfg.D + WL.window_entry_bytes(cfg, win_fmt)) if cfg.W else 0)
    scan_bytes = B * N * M.row_bytes(ir) + ab["q_idx_w"] // n_idx_layers + carried / n_idx_layers
    if pool:
        scan_bytes = None                                  # full and pool scans differ: no single figure
    scan_gbps = scan_bytes / (scan_us * 1e-6) / 1e9 if scan_bytes else None
    res.update({
        "value": 1e3 / ms_per_step,
        "unit": "layer-steps/s" if L_grp == 1 else "layer-groups/s",
        "ms_per_step": ms_per_step,
        "launch": ("HIP graph per layer cache" if graphs is not None else
                   "eager, one Python call per layer and kernel" if opt.python_group else
                   "eager, one C call per step"),
        "ms_per_step_eager": eager_ms if graphs is not None else ms_per_step,
        "config": {
            "workload": f"{cfg.name}: {cfg.desc}",
            "batch": B, "context_rows": N, "tokens": cfg.tokens, "heads": H, "qk_dim": cfg.D, "v_dim": cfg.d_v,
            "indexer": f"{cfg.H_I}x{cfg.d_I}", "top_k": k, "index_scores": "bf16" if opt.score_bf16 else "fp32",
            "window": cfg.W, "window_format": opt.win_fmt if cfg.W else None, "compress_m": opt.compress or None,
            "layers_per_step": L_grp,
            "main_row_bytes": M.row_bytes(mr), "indexer_row_bytes": M.row_bytes(ir),
            "rotated_layer_caches": n_layers, "parallelism": "single GPU",
            "candidate_pool": (f"{pool} blocks of {POOL_BLOCK} published by the Full layer, scored by the "
                               "Reindex layer") if pool else None,
        },
        "roofline": {
            "kernel": "indexer scan (k_scan_dma32; the first layer's carries the step's append)",
            "bound": "hbm",
            "achieved": scan_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": scan_gbps / HBM_PEAK_GBPS if scan_gbps else None,
            "traffic": scan_traffic(cfg) if headline and not opt.score_bf16 else None,
            "algorithmic_bytes_per_launch": scan_bytes,
            "avg_launch_us": scan_us,
            "launches_timed": n_scan,
            "timed_in": "a pass of whole steps after the timed region, every scan stamped",
        },
        "step_roofline": {
            "algorithmic_bytes_per_step": ab["total"],
            "achieved_gbps": step_gbps,
            "frac": step_gbps / HBM_PEAK_GBPS,
        },
        "per_kernel_breakdown": per_kernel,
    })
    del layers, graphs
    return res


def multi_query(args, cfg):
    """G positions of one sequence per step: append the G entries, score and select for
    the G queries in one mla_indexer_topk call over the shared cache (stride 0; query i
    sees rows < N - G + 1 + i), then one mla_sparse_decode call for the G queries."""
    import numpy as np
    import torch

    import sparse_latent_attention_mla_amd as M
    import workloads as WL

    G = args.queries
    if cfg.W or len(cfg.layers) > 1:
        raise SystemExit("--queries: single-layer configurations without a window (c2, c3, c4x)")
    cfg1 = cfg.with_(B=1)
    dev = "cuda"
    torch.cuda.set_device(0)
    n_layers = max(1, args.layers)
    log(f"multi-query {cfg.name}: one sequence of {cfg.N} rows, {G} queries per step; {n_layers} layer caches")
    layers = build_layers(cfg1, n_layers)
    N, H, k = cfg.N, cfg.H, cfg.k
    mr = M.Row(cfg.main_fmt, cfg.dim, cfg.rope)
    ir = M.Row(cfg.idx_fmt, cfg.d_I, 0)
    qdt = torch.float32 if cfg.main_fmt == WL.F32 else torch.bfloat16
    for l, X in enumerate(layers):                       # G queries, G new entries
        off = 16 * l
        X.qg = torch.from_numpy(WL.normal(0, cfg.cid, 300 + off, (G, H, cfg.D))).to(dev).to(qdt)
        X.qig = torch.from_numpy(WL.normal(0, cfg.cid, 301 + off, (G, cfg.H_I, cfg.d_I))).to(dev).to(qdt)
        X.wg = torch.from_numpy(WL.normal(0, cfg.cid, 302 + off, (G, cfg.H_I)) * np.float32(cfg.w_scale)).to(dev)
        X.newg = torch.from_numpy(WL.normal(0, cfg.cid, 303 + off, (1, G, cfg.D))).to(dev)
        X.newig = torch.from_numpy(WL.normal(0, cfg.cid, 304 + off, (1, G, cfg.d_I))).to(dev)
    slots = torch.arange(N - G, N, dtype=torch.int32, device=dev)[None].contiguous()
    nvis = torch.arange(N - G + 1, N + 1, dtype=torch.int32, device=dev)
    idx = torch.empty((G, k), dtype=torch.int32, device=dev)
    out = torch.empty((G, H, cfg.d_v), dtype=torch.float32, device=dev)
    lse = torch.empty((G, H), dtype=torch.float32, device=dev)
    ws = torch.zeros(M.mla_indexer_topk_workspace(G, N, k), dtype=torch.uint8, device=dev)
    wsd = torch.empty(max(1, M.mla_sparse_decode_workspace(mr, cfg.d_v, G, H, k, 0)), dtype=torch.uint8,
                      device=dev)

    def step(X):
        M.mla_kv_append_quant(mr, ir, X.newg, X.newig, slots, X.main, X.idx)
        M.mla_indexer_topk(ir, X.qig, X.wg, cfg.sigma, X.idx.expand(G, -1, -1), nvis, k, idx, ws,
                           score_bf16=args.score_bf16)
        M.mla_sparse_decode(mr, cfg.d_v, X.qg, X.main.expand(G, -1, -1), idx, cfg.softmax_scale, out, lse, wsd)

    for i in range(args.warmup):
        step(layers[i % n_layers])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(layers[i % n_layers])
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    M.mla_profile_enable(M.PROFILE_KERNELS)
    for i in range(min(args.steps, 50)):
        step(layers[i % n_layers])
    torch.cuda.synchronize()
    M.mla_profile_enable(())
    per_kernel = {}
    for name in M.PROFILE_KERNELS:
        n, tot = M.mla_profile_read(name)
        if n:
            per_kernel[name] = {"launches": n, "avg_us": tot * 1e3 / n}
    key_bytes = N * M.row_bytes(ir)
    scan_us = per_kernel.get("indexer_scan", {}).get("avg_us")
    log(f"{ms * 1e3:.2f} us/step for {G} queries; breakdown (avg us): " +
        ", ".join(f"{kk}={v['avg_us']:.2f}" for kk, v in per_kernel.items()))
    result = {
        "metric": METRIC + " (several queries of one sequence per step)",
        "value": 1e3 / ms, "unit": f"steps/s ({G} queries each)", "queries_per_s": G * 1e3 / ms,
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name} with one sequence and {G} queries per step (stride-0 shared cache)",
                   "queries": G, "context_rows": N, "heads": H, "top_k": k, "rotated_layer_caches": n_layers,
                   "index_scores": "bf16" if args.score_bf16 else "fp32"},
        "scan": {"key_bytes_per_launch": key_bytes, "avg_launch_us": scan_us,
                 "key_gbps_once": key_bytes / (scan_us * 1e-6) / 1e9 if scan_us else None},
        "per_kernel_breakdown": per_kernel,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline(cfg):
    """Time the CPU oracle, as it stands, on one layer-step of the same workload
    (all sequences), on all the host's cores and on one thread.  Reported beside
    the GPU, not a target."""
    import numpy as np

    import oracle as O
    import workloads as WL

    B, N = cfg.B, cfg.N
    if len(cfg.layers) > 1 or cfg.N > 262144:
        return {"value": None, "unit": "layer-steps/s", "cores": O.num_threads(), "kind": "oracle",
                "sample": "skipped for this configuration"}
    log("cpu baseline: building the oracle's caches")
    inp = WL.step_inputs(cfg, 0)
    rbm, rbi = O.row_bytes(cfg.main_fmt, cfg.dim, cfg.rope), O.row_bytes(cfg.idx_fmt, cfg.d_I, 0)
    o_main = np.zeros((B, N, rbm), np.uint8)
    o_idx = np.zeros((B, N, rbi), np.uint8)
    pre = np.tile(np.arange(N - 1, dtype=np.int32), (B, 1))
    O.append((cfg.main_fmt, cfg.dim, cfg.rope), (cfg.idx_fmt, cfg.d_I, 0), inp.main[:, :N - 1],
             inp.idx[:, :N - 1], pre, o_main, o_idx)
    last = np.full((B, 1), N - 1, np.int32)
    nvis = np.full(B, N, np.int32)

    def timed(budget_s, max_reps):
        times = []
        for rep in range(max_reps):
            t0 = time.perf_counter()
            O.append((cfg.main_fmt, cfg.dim, cfg.rope), (cfg.idx_fmt, cfg.d_I, 0), inp.main[:, N - 1:],
                     inp.idx[:, N - 1:], last, o_main, o_idx)
            s = O.indexer_scores((cfg.idx_fmt, cfg.d_I, 0), inp.q_idx[0], inp.w[0], cfg.sigma, o_idx, nvis)
            idx = O.topk(s, nvis, cfg.k)
            O.attention((cfg.main_fmt, cfg.dim, cfg.rope), cfg.d_v, inp.q[0], o_main, idx, cfg.softmax_scale)
            times.append(time.perf_counter() - t0)
            log(f"cpu baseline ({O.num_threads()} threads) rep {rep}: {times[-1]:.2f}s")
            if sum(times) > budget_s:
                break
        return times

    what = (f"full layer-steps of {cfg.name} (append + fp64 indexer scores over all {B}x{N} rows + "
            f"top-{cfg.k} + attention)")
    all_cores = O.num_threads()
    times = timed(20, 3)
    t = statistics.median(times)
    res = {"value": 1.0 / t, "unit": "layer-steps/s", "cores": all_cores, "kind": "oracle",
           "sample": f"{len(times)} {what}, median {t:.3f}s"}
    O.set_num_threads(1)
    try:
        times1 = timed(15, 2)
    finally:
        O.set_num_threads(all_cores)
    t1 = statistics.median(times1)
    res["one_thread"] = {"value": 1.0 / t1, "unit": "layer-steps/s", "cores": 1, "kind": "oracle",
                         "sample": f"{len(times1)} {what}, median {t1:.3f}s"}
    return res


if __name__ == "__main__":
    main()
