"""The layer-group helper (csa2_group_step, a composition of the C-ABI calls only)
against the same calls made one by one, and against the oracle's step: Full /
Reindex layers select with their own indexer query over the shared keys, Reuse
layers take the latest selection, every layer attends with its own query and
window ("DeepSeek-V4.1", "Three modes"; "CSA2: four layers keep their own copy").

The cases' caches already hold the step's entry (position N-1, and the window
entries of position p); the helper appends the same values to the same slots
again, which leaves every cache byte unchanged."""
import sys

import numpy as np
import pytest
import torch

import workloads as WL
from tests import gpu_cases as G
from tests.test_gpu_pool import check_pool_near, check_pool_topk

pytestmark = pytest.mark.gpu
C = WL.CONFIGS
CFGS = {
    "c1": C["c1"],
    "c3d": C["c3"].with_(name="c3d", cid=123, B=2, N=6004),
    "c4d": C["c4"].with_(name="c4d", cid=124, B=2, N=4100),
    "c5s": C["c5"].with_(name="c5s", cid=105, B=1, N=3001),
    "c5d": C["c5"].with_(name="c5d", cid=125, B=2, N=4100),
    # more rows than the one-workgroup selection takes: the many-workgroup selection, whose
    # final the group call folds into the decode
    "c3f": C["c3"].with_(name="c3f", cid=173, B=3, N=40004),
    "c4f": C["c4"].with_(name="c4f", cid=174, B=2, N=40004),
    "c5f": C["c5"].with_(name="c5f", cid=175, B=1, N=40004),
    # the bench's c3 step at full size (64 select workgroups per sequence, two splits per
    # sequence reaching the threshold bin)
    "c3full": C["c3"],
    # bf16 rows decoded 32 heads per workgroup (the paired decode finishing the selection)
    "c2full": C["c2"],
}
POOL_BLOCK = 8


def say(*a):
    print("[group-step]", *a, file=sys.stderr, flush=True)


def _inputs(case, pool_blocks):
    cfg = case.cfg
    M, dev = G.M, G.DEV
    B, N, L, k = cfg.B, cfg.N, len(cfg.layers), cfg.k
    n_idx = WL.n_indexers(cfg)
    inp = case.inp
    x = dict(
        q=torch.stack([G._q_gpu(cfg, inp.q[l]) for l in range(L)]),
        q_idx=torch.stack([G._qi_gpu(cfg, inp.q_idx[j]) for j in range(n_idx)]),
        w=G._t(inp.w),
        nvis=G._t(case.n_visible),
        new_main=G._t(inp.main[:, N - 1:]), new_idx=G._t(inp.idx[:, N - 1:]),
        slots=torch.full((B, 1), N - 1, dtype=torch.int32, device=dev),
    )
    ws = M.mla_indexer_topk_workspace(B, N, k)
    if pool_blocks:
        ws = max(ws, M.mla_indexer_pool_workspace(B, N, POOL_BLOCK))
        x["pool"] = (pool_blocks, POOL_BLOCK, torch.empty((B, N), dtype=torch.float32, device=dev),
                     torch.empty((B, pool_blocks * POOL_BLOCK), dtype=torch.int32, device=dev))
    else:
        x["pool"] = None
    x["ws"] = torch.zeros(ws, dtype=torch.uint8, device=dev)
    x["wsd"] = torch.empty(max(1, M.mla_sparse_decode_workspace(G.main_row(cfg), cfg.d_v, B, cfg.H, k, cfg.W)),
                           dtype=torch.uint8, device=dev)
    if cfg.W:
        p = cfg.tokens - 1
        x["new_win"] = G._t(inp.win[:, :, cfg.W - 1])
        x["win_pos"] = torch.full((B,), p, dtype=torch.int32, device=dev)
        x["win_len"] = G._t(case.win_len)
    return x


def _outs(cfg):
    L, B, H = len(cfg.layers), cfg.B, cfg.H
    return (torch.full((L, B, H, cfg.d_v), float("nan"), device=G.DEV),
            torch.full((L, B, H), float("nan"), device=G.DEV),
            [torch.full((B, cfg.k), -7, dtype=torch.int32, device=G.DEV) for _ in range(2)])


def _by_hand(case, x, main, idx, win):
    """The same step as individual calls, in the group's order."""
    cfg = case.cfg
    M = G.M
    mr, ir = G.main_row(cfg), G.idx_row(cfg)
    out, lse, bufs = _outs(cfg)
    pool = x["pool"]
    latest, j, attended = None, 0, []
    for l, mode in enumerate(cfg.layers):
        wargs = (x["new_win"][l], x["win_pos"], win[l]) if cfg.W else (None, None, None)
        if mode in ("full", "reindex"):
            latest = bufs[j % 2]
            scores = pool[2] if (pool is not None and mode == "full") else None
            if l == 0:
                M.mla_kv_append_quant(mr, ir, x["new_main"], x["new_idx"], x["slots"], main, idx, *wargs)
            elif cfg.W:
                M.mla_kv_append_quant(mr, ir, None, None, None, None, None, *wargs)
            M.mla_indexer_topk(ir, x["q_idx"][j], x["w"][j], cfg.sigma, idx, x["nvis"], cfg.k, latest, x["ws"],
                               out_scores=scores, cand=pool[3] if (pool is not None and mode == "reindex") else None)
            if scores is not None:
                M.mla_indexer_pool(scores, x["nvis"], pool[0], pool[3], x["ws"], block=pool[1])
            j += 1
        elif cfg.W:
            M.mla_kv_append_quant(mr, ir, None, None, None, None, None, *wargs)
        M.mla_sparse_decode(mr, cfg.d_v, x["q"][l], main, latest, cfg.softmax_scale, out[l], lse[l], x["wsd"],
                            win[l] if cfg.W else None, x["win_len"] if cfg.W else None)
        attended.append(latest.clone())
    return out, lse, attended


def _helper(case, x, main, idx, win, calls):
    cfg = case.cfg
    out, lse, bufs = _outs(cfg)
    att = G.M.csa2_group_step(G.main_row(cfg), G.idx_row(cfg), cfg.layers, main, idx, x["nvis"], cfg.k, cfg.sigma,
                              cfg.softmax_scale, x["q"], x["q_idx"], x["w"], out, lse, x["ws"], x["wsd"], bufs,
                              new_main=x["new_main"], new_idx=x["new_idx"], slots=x["slots"],
                              win_rings=win, new_win=x.get("new_win"), win_pos=x.get("win_pos"),
                              win_len=x.get("win_len"), pool=x["pool"], between_layers=calls.append)
    # each selecting layer's buffer is overwritten two selections later: keep copies
    # of what each layer attended as soon as the group is done (two buffers suffice
    # for any group with at most two selecting layers)
    return out, lse, [a.clone() for a in att]


@pytest.mark.parametrize("name,pool", [("c1", 0), ("c3d", 0), ("c4d", 0), ("c5s", 0), ("c5d", 0), ("c5d", 96)])
def test_group_helper_matches_calls_and_oracle(name, pool):
    cfg = CFGS[name]
    say(name, "pool", pool)
    case = G.build_case(cfg, seed=3)
    x = _inputs(case, pool)
    L = len(cfg.layers)
    cache = lambda: (case.g_main.clone(), case.g_idx.clone(), case.g_win.clone() if cfg.W else None)
    main_h, idx_h, win_h = cache()
    calls = []
    out_h, lse_h, att_h = _helper(case, x, main_h, idx_h, win_h, calls)
    torch.cuda.synchronize()
    pool_pos = x["pool"][3].cpu().numpy() if pool else None      # the Full layer's pool, as the helper left it
    main_m, idx_m, win_m = cache()
    out_m, lse_m, att_m = _by_hand(case, x, main_m, idx_m, win_m)
    torch.cuda.synchronize()
    assert calls == list(range(1, L)), calls
    # re-appending the step's entry leaves the caches as built
    assert torch.equal(main_h, case.g_main) and torch.equal(idx_h, case.g_idx)
    if cfg.W:
        assert torch.equal(win_h, case.g_win)
    for l in range(L):
        a, b = att_h[l].cpu().numpy(), att_m[l].cpu().numpy()
        assert np.array_equal(np.sort(a, 1), np.sort(b, 1)), l      # the same sets (order may differ)
    # the same kernels on the same sets: outputs agree to summation order
    G.check_attention(out_h.cpu().numpy().reshape(-1, cfg.H, cfg.d_v), lse_h.cpu().numpy().reshape(-1, cfg.H),
                      out_m.cpu().numpy().reshape(-1, cfg.H, cfg.d_v), lse_m.cpu().numpy().reshape(-1, cfg.H),
                      rel=1e-5)
    if pool:                                    # the pool itself, to the scores' bar
        check_pool_near(pool_pos, G.oracle_scores(case, 0), case.n_visible, pool, POOL_BLOCK)
    # against the oracle: selections of the selecting layers, attention of every layer
    j = 0
    for l, mode in enumerate(cfg.layers):
        got = att_h[l].cpu().numpy()
        if mode in ("full", "reindex"):
            if pool and mode == "reindex":       # scored over the pool the Full layer published
                check_pool_topk(got, G.oracle_scores(case, j, cand=pool_pos), pool_pos, case.n_visible, cfg.k)
            else:
                G.check_topk(got, G.oracle_scores(case, j), case.n_visible, cfg.k)
            j += 1
        else:
            assert np.array_equal(got, att_h[l - 1].cpu().numpy())
        ref_o, ref_l = G.oracle_attention(case, l, got)
        G.check_attention(out_h[l].cpu().numpy(), lse_h[l].cpu().numpy(), ref_o, ref_l)


def test_group_helper_rejects_unknown_and_leading_reuse():
    cfg = CFGS["c5s"]
    case = G.build_case(cfg, seed=3)
    x = _inputs(case, 0)
    for modes in (("full", "bogus"), ("reuse", "full")):
        out, lse, bufs = _outs(cfg.with_(layers=modes))
        with pytest.raises(ValueError):
            G.M.csa2_group_step(G.main_row(cfg), G.idx_row(cfg), modes, case.g_main.clone(), case.g_idx.clone(),
                                x["nvis"], cfg.k, cfg.sigma, cfg.softmax_scale, x["q"], x["q_idx"], x["w"], out,
                                lse, x["ws"], x["wsd"], bufs, new_main=x["new_main"], new_idx=x["new_idx"],
                                slots=x["slots"], win_rings=case.g_win.clone(), new_win=x["new_win"],
                                win_pos=x["win_pos"], win_len=x["win_len"])
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,pool,score_bf16", [("c1", 0, False), ("c3d", 0, False), ("c4d", 0, False),
                                                  ("c5s", 0, False), ("c5d", 0, False), ("c5d", 96, False),
                                                  ("c5d", 0, True), ("c3d", 0, True),
                                                  ("c3f", 0, False), ("c3f", 0, True), ("c4f", 0, False),
                                                  ("c5f", 0, False), ("c5f", 0, True), ("c5f", 96, False),
                                                  ("c3full", 0, False), ("c2full", 0, False)])
def test_native_group_step_equals_the_helper(name, pool, score_bf16, zero_keys=False, visible=None):
    """mla_csa2_group_step (one C call) against csa2_group_step (the same calls from Python):
    the caches and window rings byte for byte, the selected sets, the pool's positions, and
    the outputs (the order of a selection's positions, and with it the decode's summation
    order, may differ); every layer's decode in the call's kernel record. Where the
    selection takes its many-workgroup path (c3f, c4f, c5f without a pool), the group call
    folds the selection's final into the decode, which then writes the index set: the
    sets must still equal the final's exactly."""
    cfg = CFGS[name]
    say("native", name, "pool", pool, "bf16 scores", score_bf16, "zero keys", zero_keys)
    case = G.build_case(cfg, seed=3)
    if zero_keys:                                        # every stored key zero: every score ties
        case.g_idx.zero_()
    L = len(cfg.layers)
    runs = []
    for native in (False, True):
        x = _inputs(case, pool)
        if visible is not None:                          # per-sequence causal limits below N
            x["nvis"] = torch.tensor(visible, dtype=torch.int32, device=G.DEV)
        main, idx = case.g_main.clone(), case.g_idx.clone()
        win = case.g_win.clone() if cfg.W else None
        out, lse, bufs = _outs(cfg)
        fn = G.M.mla_csa2_group_step if native else G.M.csa2_group_step
        att = fn(G.main_row(cfg), G.idx_row(cfg), cfg.layers, main, idx, x["nvis"], cfg.k, cfg.sigma,
                 cfg.softmax_scale, x["q"], x["q_idx"], x["w"], out, lse, x["ws"], x["wsd"], bufs,
                 new_main=x["new_main"], new_idx=x["new_idx"], slots=x["slots"], win_rings=win,
                 new_win=x.get("new_win"), win_pos=x.get("win_pos"), win_len=x.get("win_len"), pool=x["pool"],
                 score_bf16=score_bf16)
        launched = G.M.mla_last_kernels()
        att = [a.clone() for a in att]
        torch.cuda.synchronize()
        runs.append((main, idx, win, out, lse, att, x["pool"][3].clone() if pool else None, launched))
    (m0, i0, w0, o0, l0, a0, p0, _), (m1, i1, w1, o1, l1, a1, p1, launched) = runs
    assert sum("k_decode" in n for n in launched) == L, launched       # one record for the whole group
    many = name.endswith(("f", "full")) or G.M.mla_get_option("topk_path") == 2
    if many and not pool:                                # folded: k_select, then the decode finishes
        assert not any("k_select_final" in n for n in launched), launched
        assert any("k_select<" in n for n in launched), launched
    assert torch.equal(m0, m1) and torch.equal(i0, i1)
    if cfg.W:
        assert torch.equal(w0.view(torch.uint8), w1.view(torch.uint8))
    for l in range(L):
        assert np.array_equal(np.sort(a0[l].cpu().numpy(), 1), np.sort(a1[l].cpu().numpy(), 1)), l
    if pool:
        pa, pb = p0.cpu().numpy(), p1.cpu().numpy()
        for b in range(cfg.B):                   # the same blocks (block order unspecified)
            blocks = lambda p: sorted(map(tuple, p[b].reshape(-1, POOL_BLOCK).tolist()))
            assert blocks(pa) == blocks(pb), b
    G.check_attention(o1.cpu().numpy().reshape(-1, cfg.H, cfg.d_v), l1.cpu().numpy().reshape(-1, cfg.H),
                      o0.cpu().numpy().reshape(-1, cfg.H, cfg.d_v), l0.cpu().numpy().reshape(-1, cfg.H), rel=1e-5)


def test_native_group_step_with_tied_scores():
    """Every stored indexer key zero, so every visible row but the step's own scores 0: the
    threshold bin holds tens of thousands of candidates (more than the decode keeps in LDS,
    so it reads them from the selection's lists) and the exact selection goes by position.
    The folded selection must still take the final's set."""
    test_native_group_step_equals_the_helper("c3f", 0, False, zero_keys=True)


def test_native_group_step_with_ragged_visibility():
    """Causal limits below the cache's rows: one sequence with fewer visible rows than k
    (every visible row selected, -1 after them), one whose limit ends inside a select
    workgroup's slice, one at full length; the finished selection against the final's."""
    test_native_group_step_equals_the_helper("c3f", 0, False, visible=[40004, 1500, 23001])


@pytest.mark.parametrize("name", ["c3d", "c5d"])
def test_native_group_step_finishes_a_forced_many_workgroup_selection(name):
    """Short sequences with the many-workgroup selection forced (topk_path = 2): a few
    select workgroups per sequence, the decode finishing their lists; against the helper,
    which runs the same selection with its final kernel."""
    with G.M.option("topk_path", 2):
        test_native_group_step_equals_the_helper(name, 0, False)
