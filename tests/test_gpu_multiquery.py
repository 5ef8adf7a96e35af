"""Several queries of one sequence in one call (multi-token prediction): the
indexer and the decode with a cache stride of 0 (every batch row reads the same
sequence's rows), each query with its own causal limit, against the oracle run
on that sequence's cache once per query."""
import numpy as np
import pytest
import torch

import workloads as WL
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
C = WL.CONFIGS
CFGS = {
    "c3s": C["c3"].with_(name="c3s", cid=103, B=2, N=6001),
    "c4s": C["c4"].with_(name="c4s", cid=104, B=2, N=4099),
    # sequences ending on a 16-byte boundary: the LDS-DMA scans read the shared rows
    "c3d": C["c3"].with_(name="c3d", cid=123, B=2, N=6004),
    "c4d": C["c4"].with_(name="c4d", cid=124, B=2, N=4100),
    "c4xd": C["c4x"].with_(name="c4xd", cid=126, B=2, N=4100),
}


@pytest.mark.parametrize("Q", [2, 3, 4, 16])
@pytest.mark.parametrize("name", sorted(CFGS))
def test_several_queries_of_one_sequence(name, Q):
    """Q positions of one sequence in one call (a prefill chunk or the drafts of
    multi-token prediction): the last Q positions, each with its causal limit, and
    for Q = 16 some much shorter limits too (ragged)."""
    cfg = CFGS[name]
    print("multi-query", name, Q, flush=True)
    case = G.build_case(cfg, seed=5)
    M, O = G.M, G.O
    N, k = cfg.N, cfg.k
    rng = np.random.default_rng(cfg.cid + 51 + Q)
    nv = np.arange(N - Q + 1, N + 1, dtype=np.int32)      # the step's positions: their causal limits
    if Q == 16:
        nv[:4] = [1, k // 3, k + 1, N // 2]
    bf = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy()   # as handed over
    q_idx = bf(rng.standard_normal((Q, cfg.H_I, cfg.d_I)))
    w = (rng.standard_normal((Q, cfg.H_I)) * cfg.w_scale).astype(np.float32)
    o_idx = np.repeat(case.o_idx[0:1], Q, axis=0)           # sequence 0's rows, once per query
    ref = O.indexer_scores((cfg.idx_fmt, cfg.d_I, 0), q_idx, w, cfg.sigma, o_idx, nv)
    out_idx = torch.empty((Q, k), dtype=torch.int32, device=G.DEV)
    scores = torch.empty((Q, N), dtype=torch.float32, device=G.DEV)
    ws = torch.zeros(M.mla_indexer_topk_workspace(Q, N, k), dtype=torch.uint8, device=G.DEV)
    shared_idx = case.g_idx[0:1].expand(Q, -1, -1)
    M.mla_indexer_topk(G.idx_row(cfg), G._qi_gpu(cfg, q_idx), G._t(w), cfg.sigma, shared_idx, G._t(nv), k,
                       out_idx, ws, out_scores=scores)
    launched = M.mla_last_kernels()
    torch.cuda.synchronize()
    if name.endswith("d"):
        assert any("k_scan_dma32" in n for n in launched), launched
        assert sum("k_scan" in n for n in launched) == 1, launched     # every query in one launch
    got_idx, got_s = out_idx.cpu().numpy(), scores.cpu().numpy()
    G.check_scores(got_s, ref, nv)
    G.check_topk(got_idx, ref, nv, k)
    # the decode of the three queries over the shared main rows, each with its own selection
    q = bf(rng.standard_normal((Q, cfg.H, cfg.D)))
    o_main = np.repeat(case.o_main[0:1], Q, axis=0)
    ref_o, ref_l = O.attention((cfg.main_fmt, cfg.dim, cfg.rope), cfg.d_v, q, o_main, got_idx, cfg.softmax_scale)
    out = torch.empty((Q, cfg.H, cfg.d_v), dtype=torch.float32, device=G.DEV)
    lse = torch.empty((Q, cfg.H), dtype=torch.float32, device=G.DEV)
    wsd = torch.empty(max(1, M.mla_sparse_decode_workspace(G.main_row(cfg), cfg.d_v, Q, cfg.H, k, 0)),
                      dtype=torch.uint8, device=G.DEV)
    M.mla_sparse_decode(G.main_row(cfg), cfg.d_v, G._q_gpu(cfg, q), case.g_main[0:1].expand(Q, -1, -1),
                        G._t(got_idx), cfg.softmax_scale, out, lse, wsd)
    torch.cuda.synchronize()
    G.check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l)


def test_padded_stride_scores_every_row():
    """A sequence stride padded to a 16-byte multiple over rows whose total is
    not one (6001 rows of 132 B): every row is scored from its own bytes, the
    last one included, as with the unpadded cache."""
    import dataclasses
    cfg = CFGS["c3s"]
    print("padded stride", flush=True)
    case = G.build_case(cfg, seed=5)
    B, N, rb = cfg.B, cfg.N, case.g_idx.shape[2]
    stride = (N * rb + 15) // 16 * 16 + 16
    buf = torch.zeros(B * stride, dtype=torch.uint8, device=G.DEV)
    view = buf.as_strided((B, N, rb), (stride, rb, 1))
    view.copy_(case.g_idx)
    padded = dataclasses.replace(case, g_idx=view)
    got_idx, got_s = G.gpu_topk(padded)
    ref = G.oracle_scores(case)
    G.check_scores(got_s, ref, case.n_visible)
    G.check_topk(got_idx, ref, case.n_visible, cfg.k)
