"""GPU parity of the HIP path against the CPU oracle, through the C ABI.

Bars (the tolerances the path is specified to):
  * quantise-append and causal masking: bit-exact;
  * indexer scores: |I_gpu - I_ref| <= 1e-4 * max(|I_ref|, rms of the row);
  * top-k sets: exact, except positions whose oracle score lies within
    1e-4 * max(|theta|, rms) of the oracle's k-th score theta;
  * attention given identical dequantised rows and index sets: per (b, h),
    max |o - o_ref| <= 2e-3 * max |o_ref| and |lse - lse_ref| <= 2e-3 * max(1, |lse_ref|).
"""
import dataclasses
import functools
import sys

import numpy as np
import pytest
import torch

import workloads as WL
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu

C = WL.CONFIGS
SMALL = {
    "c1": C["c1"],
    "c2s": C["c2"].with_(name="c2s", cid=102, B=2, N=5003),
    # bf16 rows and keys with a bf16 window ring: the bf16 scan carrying the append, window included
    "c2sw": C["c2"].with_(name="c2sw", cid=107, B=3, N=4100, W=64),
    "c3s": C["c3"].with_(name="c3s", cid=103, B=2, N=6001),
    "c4s": C["c4"].with_(name="c4s", cid=104, B=2, N=4099),
    "c4xs": C["c4x"].with_(name="c4xs", cid=106, B=2, N=5021),
    "c5s": C["c5"].with_(name="c5s", cid=105, B=1, N=3001),
    # sizes at which every wave of the queue-fed scan draws several tickets
    "c3m": C["c3"].with_(name="c3m", cid=113, B=3, N=40001),
    "c4m": C["c4"].with_(name="c4m", cid=114, B=1, N=70001),
    # sequences ending on a 16-byte boundary (N % 4 == 0) but not on a 64-row chunk:
    # the LDS-DMA scans (and the append they carry), with a ragged last chunk
    "c3d": C["c3"].with_(name="c3d", cid=123, B=2, N=6004),
    "c4d": C["c4"].with_(name="c4d", cid=124, B=2, N=4100),
    "c4xd": C["c4x"].with_(name="c4xd", cid=126, B=2, N=4100),
    # the queue-fed and static LDS-DMA scans at sizes where every wave draws several tickets
    "c3q": C["c3"].with_(name="c3q", cid=133, B=3, N=40004),
    "c4q": C["c4"].with_(name="c4q", cid=134, B=1, N=70004),
}
# the cases whose indexer cache the LDS-DMA scans read (16-byte aligned sequence ends)
DMA_CASES = ("c3d", "c4d", "c4xd")
FULL = {n: C[n] for n in ("c2", "c3", "c4", "c4x", "c5")}
TOPK_PATH = {"row": 1, "multi": 2}


def say(*a):
    print("[gpu-parity]", *a, file=sys.stderr, flush=True)


@functools.lru_cache(maxsize=4)
def case_of(name):
    cfg = SMALL.get(name) or FULL[name]
    say("building", name, f"B={cfg.B} N={cfg.N} H={cfg.H} fmt={cfg.main_fmt}/{cfg.idx_fmt} W={cfg.W}")
    return G.build_case(cfg)


def indexer_layers(cfg):
    """(layer, indexer query slot) of the layers that run the indexer."""
    out, j = [], 0
    for l, mode in enumerate(cfg.layers):
        if mode in ("full", "reindex"):
            out.append((l, j))
            j += 1
    return out


def oracle_indices_per_layer(case):
    """CSA2 composition on the oracle side: Full / Reindex layers select with
    their own indexer query over the shared keys; Reuse layers take the latest."""
    cfg = case.cfg
    idx_of, latest, j = [], None, 0
    for mode in cfg.layers:
        if mode in ("full", "reindex"):
            s = G.oracle_scores(case, j)
            latest = G.O.topk(s, case.n_visible, cfg.k)
            j += 1
        idx_of.append(latest)
    return idx_of


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


@pytest.mark.parametrize("name", list(SMALL))
def test_append_bitexact(name):
    case = case_of(name)
    say("append parity", name)
    assert np.array_equal(case.g_main.cpu().numpy(), case.o_main), "main rows differ"
    assert np.array_equal(case.g_idx.cpu().numpy(), case.o_idx), "indexer rows differ"
    if case.cfg.W:
        g = case.g_win.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(g, case.o_win), "window ring differs"


@pytest.mark.parametrize("name", list(SMALL))
def test_indexer_scores_and_topk(name):
    case = case_of(name)
    cfg = case.cfg
    for layer, j in indexer_layers(cfg):
        say("indexer", name, "layer", layer)
        got_idx, got_s = G.gpu_topk(case, j)
        ref_s = G.oracle_scores(case, j)
        G.check_scores(got_s, ref_s, case.n_visible)
        G.check_topk(got_idx, ref_s, case.n_visible, cfg.k)


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_given_oracle_indices(name):
    case = case_of(name)
    for layer, idx in enumerate(oracle_indices_per_layer(case)):
        say("decode", name, "layer", layer, case.cfg.layers[layer])
        ref_o, ref_l = G.oracle_attention(case, layer, idx)
        got_o, got_l = G.gpu_decode(case, layer, idx)
        G.check_attention(got_o, got_l, ref_o, ref_l)


@pytest.mark.parametrize("name", list(SMALL))
def test_step_end_to_end(name):
    """The GPU's own indices feed the GPU decode. Every sequence's output is
    compared with the oracle's attention over the GPU's selected set (which the
    top-k bar has already tied to the oracle's set), and where the two sets
    coincide exactly, also with the oracle's whole step."""
    case = case_of(name)
    cfg = case.cfg
    ref_idx = oracle_indices_per_layer(case)
    latest, j = None, 0
    for layer, mode in enumerate(cfg.layers):
        if mode in ("full", "reindex"):
            latest, _ = G.gpu_topk(case, j, want_scores=False)
            G.check_topk(latest, G.oracle_scores(case, j), case.n_visible, cfg.k)
            j += 1
        say("step", name, "layer", layer, mode)
        got_o, got_l = G.gpu_decode(case, layer, latest)
        own_o, own_l = G.oracle_attention(case, layer, latest)
        G.check_attention(got_o, got_l, own_o, own_l)        # all B sequences
        ref_o, ref_l = G.oracle_attention(case, layer, ref_idx[layer])
        same = 0
        for b in range(cfg.B):
            if set(latest[b].tolist()) == set(ref_idx[layer][b].tolist()):
                G.check_attention(got_o[b:b + 1], got_l[b:b + 1], ref_o[b:b + 1], ref_l[b:b + 1])
                same += 1
        say(f"  {cfg.B} sequences against the GPU's sets, {same} also against the oracle's step")


@pytest.mark.parametrize("name", ["c1", "c3s", "c4s", "c4xs"])
def test_causal_mask_and_short_contexts(name):
    case = case_of(name)
    cfg = case.cfg
    N, k = cfg.N, cfg.k
    for nv in ([0] * cfg.B, [min(N, k // 2 + 3)] + [N] * (cfg.B - 1), [N - 1] + [1] * (cfg.B - 1),
               [k] * cfg.B, [k + 1] * cfg.B):
        nv = np.array([min(v, N) for v in nv], np.int32)
        say("mask", name, nv.tolist())
        got_idx, got_s = G.gpu_topk(case, 0, n_visible=nv)
        ref_s = G.oracle_scores(case, 0, n_visible=nv)
        G.check_scores(got_s, ref_s, nv)
        G.check_topk(got_idx, ref_s, nv, k)


@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c4s"])
def test_decode_edge_cases(name):
    case = case_of(name)
    cfg = case.cfg
    rng = np.random.default_rng(7)
    B, N = cfg.B, cfg.N
    k = min(cfg.k, 300)
    idx = np.stack([rng.permutation(N)[:k] for _ in range(B)]).astype(np.int32)
    variants = {
        "ragged_minus_ones": np.where(rng.random((B, k)) < 0.3, -1, idx).astype(np.int32),
        "duplicates": np.concatenate([idx[:, :k // 2], idx[:, :k - k // 2]], 1).astype(np.int32),
        "all_minus_one": -np.ones((B, 37), np.int32),
        "single": idx[:, :1].copy(),
        "out_of_range_skipped": np.concatenate([idx[:, :50], np.full((B, 5), N + 7, np.int32)], 1),
    }
    for vname, v in variants.items():
        say("decode edge", name, vname)
        ref_v = np.where((v >= 0) & (v < N), v, -1).astype(np.int32)
        ref_o, ref_l = G.oracle_attention(case, 0, ref_v)
        got_o, got_l = G.gpu_decode(case, 0, v)
        G.check_attention(got_o, got_l, ref_o, ref_l)
    if cfg.W:
        say("decode edge", name, "window only")
        empty = np.zeros((B, 0), np.int32)
        ref_o, ref_l = G.oracle_attention(case, 0, empty)
        got_o, got_l = G.gpu_decode(case, 0, empty)
        G.check_attention(got_o, got_l, ref_o, ref_l)


@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c4s"])
def test_decode_with_attention_sinks(name):
    """Attention sinks (one logit per head in the softmax normaliser, no value
    vector): ordinary, dominant (+40: the output nearly vanishes) and absent
    (-inf) sinks, with and without the window; an empty set puts all mass on
    the sink (lse = sink, out = 0)."""
    case = case_of(name)
    cfg = case.cfg
    rng = np.random.default_rng(cfg.cid + 7)
    idx = oracle_indices_per_layer(case)[0]
    sinks = (rng.standard_normal(cfg.H) * 3).astype(np.float32)
    sinks[0], sinks[1] = 40.0, -np.inf
    for with_window in ((True, False) if cfg.W else (True,)):
        say("sinks", name, "window", with_window)
        ref_o, ref_l = G.oracle_attention(case, 0, idx, sinks=sinks, with_window=with_window)
        got_o, got_l = G.gpu_decode(case, 0, idx, with_window=with_window, sinks=sinks)
        G.check_attention(got_o, got_l, ref_o, ref_l)
    empty = -np.ones((cfg.B, 4), np.int32)
    got_o, got_l = G.gpu_decode(case, 0, empty, with_window=False, sinks=sinks)
    assert np.all(got_o == 0) and np.array_equal(got_l, np.tile(sinks, (cfg.B, 1)))


@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c4s"])
def test_decode_output_rope_inverse(name):
    """The output's RoPE inverse (the trailing r channels rotated back at each
    sequence's query position, rotate-half pairing), alone and with sinks, with
    and without the window."""
    case = case_of(name)
    cfg = case.cfg
    rng = np.random.default_rng(cfg.cid + 11)
    idx = oracle_indices_per_layer(case)[0]
    r = 16 if cfg.d_v < 128 else 64
    ang = rng.uniform(-np.pi, np.pi, (cfg.B, r // 2))
    cs = np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)
    sinks = (rng.standard_normal(cfg.H) * 2).astype(np.float32)
    for with_window in ((True, False) if cfg.W else (True,)):
        for sk in (None, sinks):
            say("output rope", name, "window", with_window, "sinks", sk is not None)
            ref_o, ref_l = G.oracle_attention(case, 0, idx, sinks=sk, with_window=with_window, rope_cs=cs)
            got_o, got_l = G.gpu_decode(case, 0, idx, with_window=with_window, sinks=sk, rope_cs=cs)
            G.check_attention(got_o, got_l, ref_o, ref_l)


@pytest.mark.parametrize("name,H", [("c2s", 16), ("c3s", 32), ("c3s", 16), ("c4s", 32), ("c5s", 16)])
def test_decode_head_counts(name, H):
    """Fewer than 64 heads: only one or two of a workgroup's waves contract while
    all of them gather; the first H heads of the configuration's queries."""
    case = case_of(name)
    sub = dataclasses.replace(case, cfg=case.cfg.with_(H=H),
                              inp=dataclasses.replace(case.inp, q=np.ascontiguousarray(case.inp.q[:, :, :H])))
    rng = np.random.default_rng(H)
    B, N, k = sub.cfg.B, sub.cfg.N, sub.cfg.k
    idx = np.stack([rng.permutation(N)[:k] for _ in range(B)]).astype(np.int32)
    idx[:, -5:] = -1
    say("decode heads", name, H)
    ref_o, ref_l = G.oracle_attention(sub, 0, idx)
    got_o, got_l = G.gpu_decode(sub, 0, idx)
    G.check_attention(got_o, got_l, ref_o, ref_l)


@pytest.mark.parametrize("path", ["row", "multi"])
@pytest.mark.parametrize("fmt", [G.O.E4M3_S128, G.O.E2M1_S16, G.O.MXFP4, G.O.BF16])
@pytest.mark.parametrize("k", [1, 37, 2048])
def test_topk_exact_ties(fmt, k, path):
    """Scores that are exact integers on both sides: integer queries and weights, and
    rows whose values the format holds exactly with unit block scales (a 448 in each
    E4M3 block of 128, a 6 in each E2M1 group of 16). Rows repeat, so many share a
    score; the selected set must equal the oracle's exactly, the smaller position
    winning each tie, and the scores must agree bit for bit. Both selection paths:
    one workgroup per sequence, and many with a separate final step."""
    rng = np.random.default_rng(1000 + 10 * fmt + k)
    B, N, d, H_I = 2, 5003, 128, 64
    distinct = rng.choice(np.array([-3, -2, -1, 0, 1, 2, 3], np.float32), (B, 997, d))
    if fmt == G.O.E4M3_S128:
        distinct[:, :, 5] = 448.0
    elif fmt in (G.O.E2M1_S16, G.O.MXFP4):                          # (MXFP4: queries of +-1 stay exact)
        distinct[:, :, ::16] = 6.0
    rows = np.ascontiguousarray(distinct[:, np.arange(N) % 997])          # each row repeats ~5 times
    q_idx = rng.choice(np.array([-1, 0, 1], np.float32), (B, H_I, d))
    w = rng.choice(np.array([1, 2], np.float32), (B, H_I))
    nv = np.array([N, N - 1234], np.int32)
    row = (fmt, d, 0)
    rb = G.O.row_bytes(fmt, d, 0)
    slots = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    o_cache = np.zeros((B, N, rb), np.uint8)
    G.O.append(row, row, None, rows, slots, None, o_cache)
    ref_s = G.O.indexer_scores(row, q_idx, w, 1.0, o_cache, nv)
    ref_i = G.O.topk(ref_s, nv, k)
    g_cache = torch.zeros((B, N, rb), dtype=torch.uint8, device="cuda")
    G.M.mla_kv_append_quant(G.M.Row(fmt, d, 0), G.M.Row(fmt, d, 0), None, G._t(rows), G._t(slots), None, g_cache)
    out_idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    out_s = torch.empty((B, N), dtype=torch.float32, device="cuda")
    ws = torch.zeros(G.M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device="cuda")
    say("topk ties", fmt, k, path)
    with G.M.option("topk_path", TOPK_PATH[path]):
        G.M.mla_indexer_topk(G.M.Row(fmt, d, 0), G._t(q_idx, torch.bfloat16), G._t(w), 1.0, g_cache, G._t(nv), k,
                             out_idx, ws, out_scores=out_s)
        launched = G.M.mla_last_kernels()
    assert any(("k_topk_row" in n) == (path == "row") for n in launched), launched
    torch.cuda.synchronize()
    got_s, got_i = out_s.cpu().numpy(), out_idx.cpu().numpy()
    for b in range(B):
        n = int(nv[b])
        assert np.array_equal(got_s[b, :n], ref_s[b, :n]), f"row {b}: scores differ"
        assert np.all(np.isneginf(got_s[b, n:]))
        assert len(np.unique(ref_s[b, :n])) < n // 4                 # the case really is full of ties
        assert np.array_equal(np.sort(got_i[b]), np.sort(ref_i[b])), f"row {b}: selected sets differ"


def test_quantise_bitexact_over_magnitudes():
    """Rows spanning 12 decades, exact zeros, signed zeros, tiny subnormal-range
    values and block maxima sitting on format boundaries, in every format."""
    rng = np.random.default_rng(11)
    n = 4096
    x = rng.standard_normal((1, n, 576)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-8, 4, (1, n, 1))).astype(np.float32)
    x[0, :16] = 0.0
    x[0, 16:32] = -0.0
    x[0, 32:48, ::3] = 448.0
    x[0, 48:64, ::5] = 6.0
    x[0, 64:80] *= np.float32(1e-30)
    x[0, 80:96, :] = rng.choice([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0], (16, 576)).astype(np.float32)
    for fmt, dim, rope in ((G.O.E4M3_S128, 512, 64), (G.O.E2M1_S16, 512, 0), (G.O.BF16, 512, 64),
                           (G.O.E4M3_S128, 128, 0), (G.O.E2M1_S16, 128, 0), (G.O.MXFP4, 128, 0),
                           (G.O.MXFP4, 512, 0), (G.O.F32, 64, 16)):
        say("quantise", fmt, dim, rope)
        D = dim + rope
        src = np.ascontiguousarray(x[:, :, :D])
        rb = G.O.row_bytes(fmt, dim, rope)
        ref = np.zeros((1, n, rb), np.uint8)
        slots = np.arange(n, dtype=np.int32)[None]
        G.O.append((fmt, dim, rope), (fmt, dim, rope), src, None, slots, ref, None)
        got = torch.zeros((1, n, rb), dtype=torch.uint8, device="cuda")
        G.M.mla_kv_append_quant(G.M.Row(fmt, dim, rope), G.M.Row(fmt, dim, 0), G._t(src), None, G._t(slots),
                                got, None)
        torch.cuda.synchronize()
        g = got.cpu().numpy()
        bad = np.flatnonzero(np.any(g != ref, axis=(0, 2)))
        assert bad.size == 0, f"fmt {fmt}: {bad.size} rows differ, first {bad[:5]}"


# ---- full sizes (the configurations the benchmark times) -----------------
@pytest.mark.parametrize("name", list(FULL))
def test_full_size(name):
    case = case_of(name)
    cfg = case.cfg
    say("full append parity", name)
    assert np.array_equal(case.g_main.cpu().numpy(), case.o_main)
    assert np.array_equal(case.g_idx.cpu().numpy(), case.o_idx)
    ref_idx = oracle_indices_per_layer(case)
    for layer, j in indexer_layers(cfg):
        say("full indexer", name, "layer", layer)
        got_idx, got_s = G.gpu_topk(case, j)
        ref_s = G.oracle_scores(case, j)
        G.check_scores(got_s, ref_s, case.n_visible)
        ne = G.check_topk(got_idx, ref_s, case.n_visible, cfg.k)
        say("  exempt boundary swaps:", ne)
    for layer in range(len(cfg.layers)):
        say("full decode", name, "layer", layer)
        ref_o, ref_l = G.oracle_attention(case, layer, ref_idx[layer])
        got_o, got_l = G.gpu_decode(case, layer, ref_idx[layer])
        wo, wl = G.check_attention(got_o, got_l, ref_o, ref_l)
        say(f"  worst rel err out {wo:.2e} lse {wl:.2e}")


def test_topk_workspace_reused_across_shapes():
    """One workspace, zeroed once, serves calls of different batch sizes,
    capacities, formats and selection paths in a row: each call must leave the
    histogram part zeroed for the next."""
    cases = [case_of(n) for n in ("c3s", "c2s", "c4s")]
    size = max(G.M.mla_indexer_topk_workspace(c.cfg.B, c.cfg.N, c.cfg.k) for c in cases)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for name, path in (("c3s", "multi"), ("c2s", "row"), ("c3s", "row"), ("c4s", "multi"), ("c3s", "multi"),
                       ("c2s", "multi")):
        case = case_of(name)
        say("workspace reuse", name, path)
        with G.M.option("topk_path", TOPK_PATH[path]):
            got_idx, _ = G.gpu_topk(case, 0, ws=ws, want_scores=False)
        ref_s = G.oracle_scores(case, 0)
        G.check_topk(got_idx, ref_s, case.n_visible, case.cfg.k)


@pytest.mark.parametrize("scan", ["queues", "static"])
@pytest.mark.parametrize("name", ["c3q", "c4q"])
def test_scan_work_queues(name, scan):
    """The queue-fed scan (chunks handed out by ticket at run time, 48 and 64
    queues here, several tickets per wave) and the statically partitioned one,
    on ragged visible lengths, with one workspace reused across the calls: the
    scores, the selection, and the zeroed start of the workspace (the queues'
    counters, then the histogram copies) after every call."""
    case = case_of(name)
    cfg = case.cfg
    B, N, k = cfg.B, cfg.N, cfg.k
    ws = torch.zeros(G.M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device="cuda")
    zero_part = 512 * 128 + B * 8 * (64 + 4096) * 4
    rng = np.random.default_rng(cfg.cid)
    for nv in ([N] * B, rng.integers(1, N + 1, B).tolist(), [N - 31] + [33] * (B - 1), [0] * B):
        nv = np.array(nv, np.int32)
        say("scan queues", name, scan, nv.tolist())
        with G.M.option("scan_queues", int(scan == "queues")):
            got_idx, got_s = G.gpu_topk(case, 0, n_visible=nv, ws=ws)
            launched = G.M.mla_last_kernels()
        want = "k_scan_dyn32" if scan == "queues" else "k_scan_dma32"
        assert any(want in n for n in launched), launched
        ref_s = G.oracle_scores(case, 0, n_visible=nv)
        G.check_scores(got_s, ref_s, nv)
        G.check_topk(got_idx, ref_s, nv, k)
        assert not bool(ws[:zero_part].any()), "workspace start not zero after the call"


@pytest.mark.parametrize("slots_kind", ["step", "spread", "tiles"])
@pytest.mark.parametrize("name", ["c3s", "c4s", "c4xs", "c3m", "c2s", "c2sw", "c1", "c3d", "c4d", "c4xd"])
def test_append_indexer_topk_equals_the_two_calls(name, slots_kind):
    """mla_append_indexer_topk against mla_kv_append_quant then mla_indexer_topk on
    copies of the same caches whose new slots hold stale bytes: the caches and the
    window ring byte for byte, the scores bit for bit, the selected sets equal; and
    against the oracle (the entries re-appended are the ones the caches were built
    from, so the expected bytes are the case's own). Entries: the step's one (slot
    N - 1), or four spread over the sequence so that several scan workgroups and
    waves each own one, or four of which three sit in the second 32-row tile of a
    64-row chunk; visible lengths that include and that exclude slot N - 1, and a
    ragged one. Where the sequences end on a 16-byte boundary, E4M3, E2M1 and MXFP4
    indexer rows take the LDS-DMA scan carrying the append, and bf16 rows the bf16 scan
    carrying it (checked by the kernel the call launched); other shapes and fp32 rows
    the separate append + scan."""
    case = case_of(name)
    cfg = case.cfg
    B, N, k = cfg.B, cfg.N, cfg.k
    mr, ir = G.main_row(cfg), G.idx_row(cfg)
    if slots_kind == "step":
        slots = [N - 1]
    elif slots_kind == "spread":
        slots = sorted({N - 1, 5 % N, N // 2, (37 * N) // 41})
    else:                                               # rows 32..63 of a 64-row chunk, and the last row
        slots = sorted({37 % N, 100 % N, (64 * (N // 128) + 50) % N, N - 1})
    sl = np.tile(np.array(slots, np.int32), (B, 1))
    new_main = G._t(case.inp.main[:, slots])
    new_idx = G._t(case.inp.idx[:, slots])
    p = cfg.tokens - 1
    posv = G._t(np.full(B, p, np.int32))
    wl0 = G._t(case.inp.win[0, :, cfg.W - 1]) if cfg.W else None

    def stale():
        m, i = case.g_main.clone(), case.g_idx.clone()
        m[:, slots] = 0xA7
        i[:, slots] = 0x5B
        wr = None
        if cfg.W:
            wr = case.g_win[0].clone()
            wr[:, p % cfg.W] = 7.0
        return m, i, wr

    for nv in ([N] * B, [N - 1] + [N] * (B - 1), [N - 70] + [max(1, N // 2 + 13)] * (B - 1)):
        nv = np.array([max(0, v) for v in nv], np.int32)
        say("append+topk", name, slots_kind, slots, nv.tolist())
        m_a, i_a, w_a = stale()
        m_b, i_b, w_b = stale()
        out_a = torch.empty((B, k), dtype=torch.int32, device="cuda")
        out_b = torch.empty_like(out_a)
        s_a = torch.empty((B, N), dtype=torch.float32, device="cuda")
        s_b = torch.empty_like(s_a)
        ws_a = torch.zeros(G.M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device="cuda")
        ws_b = torch.zeros_like(ws_a)
        qi, w = G._qi_gpu(cfg, case.inp.q_idx[0]), G._t(case.inp.w[0])
        G.M.mla_kv_append_quant(mr, ir, new_main, new_idx, G._t(sl), m_a, i_a,
                                wl0, posv if cfg.W else None, w_a)
        G.M.mla_indexer_topk(ir, qi, w, cfg.sigma, i_a, G._t(nv), k, out_a, ws_a, out_scores=s_a)
        G.M.mla_append_indexer_topk(mr, ir, new_main, new_idx, G._t(sl), m_b, i_b, qi, w, cfg.sigma, G._t(nv),
                                    k, out_b, ws_b, new_win=wl0, win_pos=posv if cfg.W else None, win_ring=w_b,
                                    out_scores=s_b)
        launched = G.M.mla_last_kernels()
        torch.cuda.synchronize()
        scans = [n for n in launched if "k_scan" in n]
        assert len(scans) == 1, launched
        if name in DMA_CASES:                           # one launch before the selection: the DMA scan carrying the append
            assert not any("k_append" in n for n in launched), launched
            assert "k_scan_dma32" in scans[0] and "true>(" in scans[0], launched
        elif name in ("c3s", "c4s", "c4xs", "c3m"):     # odd sequence ends: separate append, staged scan
            assert any("k_append" in n for n in launched) and "k_scan_staged" in scans[0], launched
        elif name in ("c2s", "c2sw"):                   # bf16 rows: the bf16 scan carrying the append
            assert not any("k_append" in n for n in launched), launched
            assert "k_scan_bf16" in scans[0] and "true>(" in scans[0], launched
        assert torch.equal(m_a, m_b) and torch.equal(i_a, i_b), "caches differ between the paths"
        assert torch.equal(i_b, case.g_idx) and torch.equal(m_b, case.g_main), "caches differ from the case's"
        if cfg.W:
            assert torch.equal(w_a.view(torch.int16), w_b.view(torch.int16))
            assert torch.equal(w_b.view(torch.int16), case.g_win[0].view(torch.int16))
        ga, gb = s_a.cpu().numpy(), s_b.cpu().numpy()
        assert np.array_equal(ga.view(np.uint32), gb.view(np.uint32)), "scores differ bit-wise"
        oa, ob = out_a.cpu().numpy(), out_b.cpu().numpy()
        for bb in range(B):
            assert set(oa[bb].tolist()) == set(ob[bb].tolist())
        ref_s = G.oracle_scores(case, 0, n_visible=nv)
        G.check_scores(gb, ref_s, nv)
        G.check_topk(ob, ref_s, nv, k)
