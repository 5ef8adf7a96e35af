"""Decode hot-path benchmark on one MI355X.

One step = one decode layer-step of the whole batch: quantise-append of the
new entry and indexer key, lightning-indexer scan + causal mask + top-k, and
sparse absorbed-MLA decode (+ window branch).  The CSA2 group configuration
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
    p.add_argument("--config", default="c3", choices=["c1", "c2", "c3", "c4", "c5"])
    p.add_argument("--layers", type=int, default=8, help="distinct layer caches rotated")
    p.add_argument("--no-cpu-baseline", action="store_true")
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
        chunk = max(1, (1 << 26) // (N * D))          # sequences per generation chunk
        for b0 in range(0, B, chunk):
            b1 = min(B, b0 + chunk)
            # positions of sequences b0..b1 in the [B, N(, m), D] streams
            if cfg.m == 1:
                main = WL.normal(seed, cfg.cid, WL.T_MAIN + off, (b1 - b0, N, D), offset=b0 * N * D)
                idx = WL.normal(seed, cfg.cid, WL.T_IDX + off, (b1 - b0, N, cfg.d_I), offset=b0 * N * cfg.d_I)
            else:
                tok = WL.normal(seed, cfg.cid, WL.T_MAIN + off, (b1 - b0, N, cfg.m, D), offset=b0 * N * cfg.m * D)
                main = tok[:, :, 0].copy()
                for jj in range(1, cfg.m):
                    main += tok[:, :, jj]
                main *= np.float32(1.0 / cfg.m)
                del tok
                tok = WL.normal(seed, cfg.cid, WL.T_IDX + off, (b1 - b0, N, cfg.m, cfg.d_I),
                                offset=b0 * N * cfg.m * cfg.d_I)
                idx = tok[:, :, 0].copy()
                for jj in range(1, cfg.m):
                    idx += tok[:, :, jj]
                idx *= np.float32(1.0 / cfg.m)
                del tok
            M.mla_kv_append_quant(mr, ir, torch.from_numpy(np.ascontiguousarray(main)).to(dev),
                                  torch.from_numpy(np.ascontiguousarray(idx)).to(dev),
                                  slots_all[b0:b1].contiguous(), X.main[b0:b1], X.idx[b0:b1])
            del main, idx
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the decode path runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_latent_attention_mla_amd as M
    import workloads as WL

    cfg = WL.CONFIGS[args.config]
    dev = "cuda"
    torch.cuda.set_device(0)
    B, N, H = cfg.B, cfg.N, cfg.H
    mr = M.Row(cfg.main_fmt, cfg.dim, cfg.rope)
    ir = M.Row(cfg.idx_fmt, cfg.d_I, 0)
    n_layers = max(1, args.layers)
    log(f"config {cfg.name}: {cfg.desc}; building {n_layers} layer caches")
    layers = build_layers(cfg, n_layers)

    # step buffers
    k = cfg.k
    nvis = torch.full((B,), N, dtype=torch.int32, device=dev)
    slots = torch.full((B, 1), N - 1, dtype=torch.int32, device=dev)
    p = cfg.tokens - 1
    win_pos = torch.full((B,), p, dtype=torch.int32, device=dev)
    win_len = torch.full((B,), min(cfg.W, p + 1), dtype=torch.int32, device=dev)
    idx_out = [torch.empty((B, k), dtype=torch.int32, device=dev) for _ in range(2)]
    out = torch.empty((B, H, cfg.d_v), dtype=torch.float32, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws_topk = torch.empty(M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(max(1, M.mla_sparse_decode_workspace(mr, cfg.d_v, B, H, k, cfg.W)), dtype=torch.uint8,
                         device=dev)
    stream = torch.cuda.current_stream()

    def step(X, ev=None):
        """One layer-step (or CSA2 group) on layer caches X.  ev: 4 events bracketing
        append / indexer / decode of the first layer of the step."""
        j = 0
        latest = None
        for l, mode in enumerate(cfg.layers):
            first = l == 0
            if ev is not None and first:
                ev[0].record(stream)
            M.mla_kv_append_quant(mr, ir, X.new_main if first else None, X.new_idx if first else None,
                                  slots if first else None, X.main if first else None, X.idx if first else None,
                                  X.new_win[l] if cfg.W else None, win_pos if cfg.W else None,
                                  X.win[l] if cfg.W else None)
            if ev is not None and first:
                ev[1].record(stream)
            if mode in ("full", "reindex"):
                latest = idx_out[j % 2]
                M.mla_indexer_topk(ir, X.q_idx[j], X.w[j], cfg.sigma, X.idx, nvis, k, latest, ws_topk)
                j += 1
            if ev is not None and first:
                ev[2].record(stream)
            M.mla_sparse_decode(mr, cfg.d_v, X.q[l], X.main, latest, cfg.softmax_scale, out, lse, ws_dec,
                                X.win[l] if cfg.W else None, win_len if cfg.W else None)
            if ev is not None and first:
                ev[3].record(stream)

    log(f"warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(layers[i % n_layers])
    torch.cuda.synchronize()

    # timed region: exactly K steps, events on the launch stream
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(layers[i % n_layers], evs[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    per_call = {
        "append": statistics.mean(e[0].elapsed_time(e[1]) for e in evs) * 1e3,
        "indexer_topk": statistics.mean(e[1].elapsed_time(e[2]) for e in evs) * 1e3,
        "sparse_decode": statistics.mean(e[2].elapsed_time(e[3]) for e in evs) * 1e3,
    }
    log(f"{ms_per_step * 1e3:.2f} us/step; per call (us): " + ", ".join(f"{k}={v:.2f}" for k, v in per_call.items()))

    ab = WL.algorithmic_bytes(cfg)
    step_gbps = ab["total"] / (ms_per_step * 1e-3) / 1e9
    # dominant call: the indexer (scan of every visible indexer row + top-k); for the
    # CSA2 group the timed bracket covers its first (Full) layer
    n_idx_layers = WL.n_indexers(cfg)
    idx_bytes = (ab["scan"] + ab["q_idx_w"]) // n_idx_layers + B * k * 4
    idx_gbps = idx_bytes / (per_call["indexer_topk"] * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": 1e3 / ms_per_step,
        "unit": "layer-steps/s" if len(cfg.layers) == 1 else "layer-groups/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.desc}",
            "batch": B, "context_rows": N, "tokens": cfg.tokens, "heads": H, "qk_dim": cfg.D, "v_dim": cfg.d_v,
            "indexer": f"{cfg.H_I}x{cfg.d_I}", "top_k": k, "window": cfg.W, "layers_per_step": len(cfg.layers),
            "main_row_bytes": M.row_bytes(mr), "indexer_row_bytes": M.row_bytes(ir),
            "rotated_layer_caches": n_layers, "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": "mla_indexer_topk (indexer scan + top-k select)",
            "bound": "hbm",
            "achieved": idx_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": idx_gbps / HBM_PEAK_GBPS,
            "traffic": None,
            "algorithmic_bytes_per_launch": idx_bytes,
            "avg_launch_us": per_call["indexer_topk"],
        },
        "step_roofline": {
            "algorithmic_bytes_per_step": ab["total"],
            "achieved_gbps": step_gbps,
            "frac": step_gbps / HBM_PEAK_GBPS,
        },
        "per_call_us": per_call,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(result), flush=True)


def cpu_baseline(cfg):
    """Time the CPU oracle, as it stands, on one layer-step of the same workload
    (all sequences), on the host's cores.  Reported beside the GPU, not a target."""
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
    times = []
    for rep in range(3):
        t0 = time.perf_counter()
        O.append((cfg.main_fmt, cfg.dim, cfg.rope), (cfg.idx_fmt, cfg.d_I, 0), inp.main[:, N - 1:],
                 inp.idx[:, N - 1:], last, o_main, o_idx)
        s = O.indexer_scores((cfg.idx_fmt, cfg.d_I, 0), inp.q_idx[0], inp.w[0], cfg.sigma, o_idx, nvis)
        idx = O.topk(s, nvis, cfg.k)
        O.attention((cfg.main_fmt, cfg.dim, cfg.rope), cfg.d_v, inp.q[0], o_main, idx, cfg.softmax_scale)
        times.append(time.perf_counter() - t0)
        log(f"cpu baseline rep {rep}: {times[-1]:.2f}s")
        if sum(times) > 30:
            break
    t = statistics.median(times)
    return {"value": 1.0 / t, "unit": "layer-steps/s", "cores": O.num_threads(), "kind": "oracle",
            "sample": f"{len(times)} full layer-steps of {cfg.name} (append + fp64 indexer scores over all "
                      f"{B}x{N} rows + top-{cfg.k} + attention), median {t:.3f}s"}


if __name__ == "__main__":
    main()
