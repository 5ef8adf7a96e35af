"""The bf16-score top-k on the GPU (mla_indexer_topk_bf16, and the fused
append + top-k) against the oracle's: the scores rounded to bf16 (round to
nearest even) and ordered by (score desc, position asc), [P1] "DeepSeek-V4",
"The indexer in four bits".

Bars (the reading of the fp32 bars for bf16 scores): the GPU's fp32 score is
within the score bar (1e-4 relative, floored at the row's rms) of the oracle's,
so its bf16 score is the rounding of some value in that bar. Rows whose range
of such roundings stays above (below) the oracle's k-th bf16 score are in
(out of) the set as the oracle's are; the sets are equal outright when every
row whose range reaches that score rounds to it alone; otherwise they may
differ among those boundary rows only."""
import numpy as np
import pytest
import torch

import workloads as WL
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
C = WL.CONFIGS
CASES = {
    "c1": C["c1"],
    "c3s": C["c3"].with_(name="c3s", cid=103, B=2, N=6001),
    "c3d": C["c3"].with_(name="c3d", cid=123, B=2, N=6004),
    "c4d": C["c4"].with_(name="c4d", cid=124, B=2, N=4100),
    "c4xd": C["c4x"].with_(name="c4xd", cid=126, B=2, N=4100),
    "c5s": C["c5"].with_(name="c5s", cid=105, B=1, N=3001),
    "c4": C["c4"],
    "c5": C["c5"],
}


def check_bf16(got_idx, got_s, o32, n_visible, k, rel=1e-4):
    """Scores and selection against the oracle's fp32 scores o32 (see the module doc):
    each GPU bf16 score must be the rounding of some value within the fp32 score bar of
    the oracle's score; rows whose range of such roundings does not reach the oracle's
    k-th bf16 score theta are in or out of the set as the oracle's are, and the sets
    are equal outright when every row whose range reaches theta rounds to theta alone.
    Returns the number of rows whose bf16 score differs from the oracle's."""
    o16 = G.O.bf16_scores(o32)
    n_mis = 0
    for b in range(o32.shape[0]):
        nv = int(n_visible[b])
        g, r16, r32 = got_s[b, :nv], o16[b, :nv], o32[b, :nv].astype(np.float64)
        assert np.all(np.isneginf(got_s[b, nv:]))
        assert np.all(g.view(np.uint32) & 0xFFFF == 0), "scores not bf16 values"
        if nv == 0:
            assert np.all(got_idx[b] < 0)
            continue
        rms = np.sqrt(np.mean(r32 * r32))
        bar = rel * np.maximum(np.abs(r32), rms)
        lo = G.O.bf16_scores((r32 - bar).astype(np.float32))
        hi = G.O.bf16_scores((r32 + bar).astype(np.float32))
        assert np.all((g >= lo) & (g <= hi)), f"row {b}: a bf16 score outside its bar"
        n_mis += int(np.sum(g != r16))
        # selection
        want = min(k, nv)
        sel = got_idx[b][got_idx[b] >= 0]
        assert np.sum(got_idx[b] < 0) == k - want and len(np.unique(sel)) == len(sel) and np.all(sel < nv)
        if want == 0:
            continue
        order = np.lexsort((np.arange(nv), -r16.astype(np.float64)))
        theta = r16[order[want - 1]]
        boundary = (lo <= theta) & (hi >= theta)
        ref = np.zeros(nv, bool)
        ref[order[:want]] = True
        gotm = np.zeros(nv, bool)
        gotm[sel] = True
        if np.all(lo[boundary] == hi[boundary]):
            assert np.array_equal(ref, gotm), f"row {b}: selected set differs"
        else:
            assert not np.any((ref != gotm) & ~boundary), f"row {b}: differences away from the boundary"
    return n_mis


def _layers(cfg):
    out, j = [], 0
    for mode in cfg.layers:
        if mode in ("full", "reindex"):
            out.append(j)
            j += 1
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_bf16_score_topk(name):
    cfg = CASES[name]
    print("bf16 scores", name, flush=True)
    case = G.build_case(cfg)
    B, N, k = cfg.B, cfg.N, cfg.k
    for j in _layers(cfg):
        out_idx = torch.empty((B, k), dtype=torch.int32, device=G.DEV)
        scores = torch.empty((B, N), dtype=torch.float32, device=G.DEV)
        ws = torch.zeros(G.M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device=G.DEV)
        G.M.mla_indexer_topk(G.idx_row(cfg), G._qi_gpu(cfg, case.inp.q_idx[j]), G._t(case.inp.w[j]), cfg.sigma,
                             case.g_idx, G._t(case.n_visible), k, out_idx, ws, out_scores=scores, score_bf16=True)
        torch.cuda.synchronize()
        o32 = G.oracle_scores(case, j)
        n_mis = check_bf16(out_idx.cpu().numpy(), scores.cpu().numpy(), o32, case.n_visible, k)
        print(f"  layer {j}: {n_mis} rows round to the neighbouring bf16 value", flush=True)
        if j == 0 and cfg.N <= 8192:                        # masked and short contexts
            nv = np.array([min(N, k // 2 + 3)] + [N - 1] * (B - 1), np.int32)
            G.M.mla_indexer_topk(G.idx_row(cfg), G._qi_gpu(cfg, case.inp.q_idx[0]), G._t(case.inp.w[0]), cfg.sigma,
                                 case.g_idx, G._t(nv), k, out_idx, ws, out_scores=scores, score_bf16=True)
            torch.cuda.synchronize()
            check_bf16(out_idx.cpu().numpy(), scores.cpu().numpy(), G.oracle_scores(case, 0, n_visible=nv), nv, k)


@pytest.mark.parametrize("name", ["c3d", "c4d"])
def test_bf16_score_topk_fused_with_the_append(name):
    """mla_append_indexer_topk_bf16 selects as mla_indexer_topk_bf16 after the append
    (the LDS-DMA scan carrying the append): the same scores bit for bit, the same set."""
    cfg = CASES[name]
    case = G.build_case(cfg)
    B, N, k = cfg.B, cfg.N, cfg.k
    mr, ir = G.main_row(cfg), G.idx_row(cfg)
    sl = G._t(np.full((B, 1), N - 1, np.int32))
    qi, w, nv = G._qi_gpu(cfg, case.inp.q_idx[0]), G._t(case.inp.w[0]), G._t(case.n_visible)
    res = []
    for fused in (False, True):
        m, i = case.g_main.clone(), case.g_idx.clone()
        out = torch.empty((B, k), dtype=torch.int32, device=G.DEV)
        sc = torch.empty((B, N), dtype=torch.float32, device=G.DEV)
        ws = torch.zeros(G.M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device=G.DEV)
        nm, ni = G._t(case.inp.main[:, N - 1:]), G._t(case.inp.idx[:, N - 1:])
        if fused:
            G.M.mla_append_indexer_topk(mr, ir, nm, ni, sl, m, i, qi, w, cfg.sigma, nv, k, out, ws, out_scores=sc,
                                        score_bf16=True)
            assert any("k_scan_dma32" in x and "true>(" in x for x in G.M.mla_last_kernels())
        else:
            G.M.mla_kv_append_quant(mr, ir, nm, ni, sl, m, i)
            G.M.mla_indexer_topk(ir, qi, w, cfg.sigma, i, nv, k, out, ws, out_scores=sc, score_bf16=True)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), sc.cpu().numpy()))
    assert np.array_equal(res[0][1].view(np.uint32), res[1][1].view(np.uint32))
    for b in range(B):
        assert set(res[0][0][b].tolist()) == set(res[1][0][b].tolist())
    check_bf16(res[1][0], res[1][1], G.oracle_scores(case, 0), case.n_visible, k)


@pytest.mark.parametrize("path", [1, 2])
def test_bf16_score_topk_exact_ties(path):
    """Integer scores (exact in bf16 and fp32 on both sides), rows repeating: the set
    must equal the oracle's exactly on both selection paths, smaller positions winning."""
    rng = np.random.default_rng(77)
    B, N, d, H_I, k = 2, 5003, 128, 64, 300
    fmt = G.O.E4M3_S128
    distinct = rng.choice(np.array([-3, -2, -1, 0, 1, 2, 3], np.float32), (B, 997, d))
    distinct[:, :, 5] = 448.0
    rows = np.ascontiguousarray(distinct[:, np.arange(N) % 997])
    q_idx = rng.choice(np.array([-1, 0, 1], np.float32), (B, H_I, d))
    w = rng.choice(np.array([1, 2], np.float32), (B, H_I))
    nv = np.array([N, N - 1234], np.int32)
    row = (fmt, d, 0)
    o_cache = np.zeros((B, N, 132), np.uint8)
    slots = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    G.O.append(row, row, None, rows, slots, None, o_cache)
    ref_s = G.O.indexer_scores(row, q_idx, w, 1.0, o_cache, nv)
    ref_i = G.O.topk_bf16(ref_s, nv, k)
    g_cache = torch.zeros((B, N, 132), dtype=torch.uint8, device=G.DEV)
    G.M.mla_kv_append_quant(G.M.Row(*row), G.M.Row(*row), None, G._t(rows), G._t(slots), None, g_cache)
    out_idx = torch.empty((B, k), dtype=torch.int32, device=G.DEV)
    ws = torch.zeros(G.M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device=G.DEV)
    with G.M.option("topk_path", path):
        G.M.mla_indexer_topk(G.M.Row(*row), G._t(q_idx, torch.bfloat16), G._t(w), 1.0, g_cache, G._t(nv), k,
                             out_idx, ws, score_bf16=True)
    torch.cuda.synchronize()
    got = out_idx.cpu().numpy()
    for b in range(B):
        assert np.array_equal(np.sort(got[b]), np.sort(ref_i[b])), f"row {b}"
