"""mla_sparse_decode_noalloc (the decode for callers that cannot allocate: the
library's static per-GPU scratch instead of a workspace) against
mla_sparse_decode on the same inputs, through the C ABI: two calls in a row, the
second with a smaller input, outputs equal bit for bit (the same kernels) and
within the attention bar of the oracle; the MXFP8 window's copy also lives in
the scratch; shapes beyond the scratch are rejected on the host."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as WL
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
C = WL.CONFIGS


def _both(case, idx, H=None, use_window=True):
    cfg = case.cfg
    M = G.M
    B = cfg.B
    H = cfg.H if H is None else H
    q = G._q_gpu(cfg, case.inp.q[0][:, :H])
    k = idx.shape[1]
    win = case.g_win[0] if (use_window and cfg.W) else None
    wl = G._t(case.win_len) if win is not None else None
    res = []
    for noalloc in (False, True):
        out = torch.full((B, H, cfg.d_v), np.nan, dtype=torch.float32, device=G.DEV)
        lse = torch.full((B, H), np.nan, dtype=torch.float32, device=G.DEV)
        if noalloc:
            M.mla_sparse_decode_noalloc(G.main_row(cfg), cfg.d_v, q, case.g_main, G._t(idx), cfg.softmax_scale,
                                        out, lse, win, wl)
        else:
            wfmt = M.MXFP8 if (win is not None and win.dtype == torch.uint8) else M.BF16
            n = M.mla_sparse_decode_workspace(G.main_row(cfg), cfg.d_v, B, H, k, cfg.W if win is not None else 0,
                                              wfmt)
            ws = torch.empty(max(n, 1), dtype=torch.uint8, device=G.DEV)
            M.mla_sparse_decode(G.main_row(cfg), cfg.d_v, q, case.g_main, G._t(idx), cfg.softmax_scale, out, lse,
                                ws, win, wl)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    return res


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_noalloc_decode_equals_the_workspace_decode(name):
    big = C[name].with_(name=f"{name}na", cid=140 + int(name[1]), B=4, N=6004)
    small = C[name].with_(name=f"{name}nb", cid=150 + int(name[1]), B=2, N=3000)
    for cfg, kk in ((big, big.k), (small, 300)):
        print("noalloc", cfg.name, cfg.B, cfg.N, kk, flush=True)
        case = G.build_case(cfg)
        rng = np.random.default_rng(cfg.cid)
        idx = np.stack([rng.permutation(cfg.N)[:kk] for _ in range(cfg.B)]).astype(np.int32)
        idx[:, -7:] = -1
        (o_ws, l_ws), (o_na, l_na) = _both(case, idx)
        assert np.array_equal(o_ws, o_na) and np.array_equal(l_ws, l_na), "differs from mla_sparse_decode"
        ref_o, ref_l = G.oracle_attention(case, 0, idx)
        G.check_attention(o_na, l_na, ref_o, ref_l)


def test_noalloc_decode_mxfp8_window_in_the_scratch():
    cfg = C["c4"].with_(name="c4nw", cid=161, B=3, N=2500)
    print("noalloc mxfp8 window", flush=True)
    case = G.build_case(cfg)
    # the window ring as MXFP8 entries of the same values
    M = G.M
    B, W, D = cfg.B, cfg.W, cfg.D
    ring8 = torch.zeros((B, W, D + D // 32), dtype=torch.uint8, device=G.DEV)
    for s in range(W):
        M.mla_kv_append_quant(G.main_row(cfg), G.idx_row(cfg), None, None, None, None, None,
                              case.g_win[0][:, s].float().contiguous(),
                              torch.full((B,), s, dtype=torch.int32, device=G.DEV), ring8)
    torch.cuda.synchronize()
    case8 = dataclasses.replace(case, g_win=torch.stack([ring8] * case.g_win.shape[0]))
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(cfg.N)[:cfg.k] for _ in range(B)]).astype(np.int32)
    (o_ws, l_ws), (o_na, l_na) = _both(case8, idx)
    assert np.array_equal(o_ws, o_na) and np.array_equal(l_ws, l_na)


def test_noalloc_rejects_shapes_beyond_the_scratch():
    M = G.M
    row = M.Row(M.E4M3_S128, 512, 64)
    B, H, k = 64, 128, 2048
    need = M.mla_sparse_decode_workspace(row, 512, B, H, k, 0)
    assert need > (32 << 20)
    q = torch.zeros((B, H, 576), dtype=torch.bfloat16, device=G.DEV)
    cache = torch.zeros((B, 8, 656), dtype=torch.uint8, device=G.DEV)
    idx = torch.zeros((B, k), dtype=torch.int32, device=G.DEV)
    out = torch.zeros((B, H, 512), dtype=torch.float32, device=G.DEV)
    lse = torch.zeros((B, H), dtype=torch.float32, device=G.DEV)
    with pytest.raises(M.MLAError, match="scratch"):
        M.mla_sparse_decode_noalloc(row, 512, q, cache, idx, 0.07, out, lse)
    assert M.mla_last_kernels() == []
