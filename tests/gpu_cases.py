"""Build one decode step of a configuration on both sides from the same seeded
inputs: the oracle (numpy + oracle/) and the HIP library (torch GPU tensors).

Each side quantises the caches with its own code; nothing computed by the HIP
path is fed to the oracle.  The GPU side may be fed oracle-chosen indices
(decode parity given identical index sets).
"""
import dataclasses
from typing import Optional

import numpy as np
import torch

import oracle as O
import sparse_latent_attention_mla_amd as M
import workloads as WL

DEV = "cuda"


def main_row(cfg):
    return M.Row(cfg.main_fmt, cfg.dim, cfg.rope)


def idx_row(cfg):
    return M.Row(cfg.idx_fmt, cfg.d_I, 0)


def _t(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    return t if dtype is None else t.to(dtype)


def _q_gpu(cfg, x):
    """Queries are handed to the GPU in bf16 (fp32 for the fp32 configuration);
    x already holds bf16-representable values in that case."""
    return _t(x, torch.float32 if cfg.main_fmt == O.F32 else torch.bfloat16)


def _qi_gpu(cfg, x):
    return _t(x, torch.float32 if cfg.idx_fmt == O.F32 else torch.bfloat16)


@dataclasses.dataclass
class Case:
    cfg: WL.Config
    inp: WL.StepInputs
    # oracle side
    o_main: np.ndarray              # uint8 [B, N, rb]
    o_idx: np.ndarray               # uint8 [B, N, rbi]
    o_win: Optional[np.ndarray]     # uint16 [L, B, W, D] or None
    # GPU side
    g_main: torch.Tensor
    g_idx: torch.Tensor
    g_win: Optional[torch.Tensor]   # bf16 [L, B, W, D]
    win_len: np.ndarray             # int32 [B]

    @property
    def n_visible(self):
        return np.full(self.cfg.B, self.cfg.N, np.int32)


COMPRESS_EPS = 1e-6


def pooled_inputs(cfg: WL.Config, seed: int = 0) -> WL.StepInputs:
    """The step inputs, with m > 1 the main entries pooled from the workload's tokens by the
    oracle's CSA2 compressor (unit norm weight, no rotation); both sides then append the
    same fp32 entries."""
    inp = WL.step_inputs(cfg, seed)
    if inp.main is not None:
        return inp
    main = np.empty((cfg.B, cfg.N, cfg.D), np.float32)
    chunk = 16384
    for b in range(cfg.B):
        for n0 in range(0, cfg.N, chunk):
            n1 = min(cfg.N, n0 + chunk)
            kv, gate = WL.compressor_tokens(cfg, seed, b, n0, n1)
            main[b, n0:n1] = O.compress(kv, gate, None, COMPRESS_EPS)
    return dataclasses.replace(inp, main=main)


def build_case(cfg: WL.Config, seed: int = 0) -> Case:
    """Caches hold positions 0..N-2 (bulk append), then the step appends
    position N-1 (n_new = 1) on each side; window rings hold the W most recent
    window entries, the last one written by the step's append."""
    inp = pooled_inputs(cfg, seed)
    B, N, D = cfg.B, cfg.N, cfg.D
    mr, ir = main_row(cfg), idx_row(cfg)
    rb, rbi = O.row_bytes(cfg.main_fmt, cfg.dim, cfg.rope), O.row_bytes(cfg.idx_fmt, cfg.d_I, 0)
    # ---- oracle
    o_main = np.zeros((B, N, rb), np.uint8)
    o_idx = np.zeros((B, N, rbi), np.uint8)
    pre = np.tile(np.arange(N - 1, dtype=np.int32), (B, 1))
    O.append((cfg.main_fmt, cfg.dim, cfg.rope), (cfg.idx_fmt, cfg.d_I, 0), inp.main[:, :N - 1],
             inp.idx[:, :N - 1], pre, o_main, o_idx)
    last = np.full((B, 1), N - 1, np.int32)
    # ---- GPU
    g_main = torch.zeros((B, N, rb), dtype=torch.uint8, device=DEV)
    g_idx = torch.zeros((B, N, rbi), dtype=torch.uint8, device=DEV)
    if N > 1:
        M.mla_kv_append_quant(mr, ir, _t(inp.main[:, :N - 1]), _t(inp.idx[:, :N - 1]), _t(pre), g_main, g_idx)
    o_win = g_win = None
    L = len(cfg.layers)
    p = cfg.tokens - 1                               # position of the current token
    win_len = np.full(B, min(cfg.W, p + 1), np.int32)
    if cfg.W:
        o_win = np.zeros((L, B, cfg.W, D), np.uint16)
        g_win = torch.zeros((L, B, cfg.W, D), dtype=torch.bfloat16, device=DEV)
        for l in range(L):
            # earlier window entries of positions p-W+1 .. p-1
            for i in range(cfg.W - 1):
                pos = p - (cfg.W - 1) + i
                if pos < 0:
                    continue
                posv = np.full(B, pos, np.int32)
                O.append((cfg.main_fmt, cfg.dim, cfg.rope), (cfg.idx_fmt, cfg.d_I, 0), None, None,
                         np.zeros((B, 0), np.int32), None, None, inp.win[l, :, i], posv, o_win[l])
                M.mla_kv_append_quant(mr, ir, None, None, None, None, None, _t(inp.win[l, :, i]),
                                      _t(posv), g_win[l])
    # ---- the step's append: entry N-1 (+ window entry of position p for layer 0)
    posv = np.full(B, p, np.int32)
    wl0 = inp.win[0, :, cfg.W - 1] if cfg.W else None
    O.append((cfg.main_fmt, cfg.dim, cfg.rope), (cfg.idx_fmt, cfg.d_I, 0), inp.main[:, N - 1:],
             inp.idx[:, N - 1:], last, o_main, o_idx,
             wl0, posv if cfg.W else None, o_win[0] if cfg.W else None)
    M.mla_kv_append_quant(mr, ir, _t(inp.main[:, N - 1:]), _t(inp.idx[:, N - 1:]), _t(last), g_main, g_idx,
                          _t(wl0) if cfg.W else None, _t(posv) if cfg.W else None,
                          g_win[0] if cfg.W else None)
    for l in range(1, L if cfg.W else 0):           # window-only appends of the other layers
        O.append((cfg.main_fmt, cfg.dim, cfg.rope), (cfg.idx_fmt, cfg.d_I, 0), None, None,
                 np.zeros((B, 0), np.int32), None, None, inp.win[l, :, cfg.W - 1], posv, o_win[l])
        M.mla_kv_append_quant(mr, ir, None, None, None, None, None, _t(inp.win[l, :, cfg.W - 1]),
                              _t(posv), g_win[l])
    torch.cuda.synchronize()
    return Case(cfg, inp, o_main, o_idx, o_win, g_main, g_idx, g_win, win_len)


# ---- oracle views -------------------------------------------------------
def oracle_scores(case: Case, layer_idx: int = 0, n_visible=None, cand=None):
    cfg = case.cfg
    nv = case.n_visible if n_visible is None else n_visible
    return O.indexer_scores((cfg.idx_fmt, cfg.d_I, 0), case.inp.q_idx[layer_idx], case.inp.w[layer_idx],
                            cfg.sigma, case.o_idx, nv, cand=cand)


def oracle_attention(case: Case, layer: int, idx: np.ndarray, sinks=None, with_window=True, rope_cs=None):
    cfg = case.cfg
    use_w = with_window and cfg.W > 0
    win = case.o_win[layer] if use_w else None
    return O.attention((cfg.main_fmt, cfg.dim, cfg.rope), cfg.d_v, case.inp.q[layer], case.o_main, idx,
                       cfg.softmax_scale, win, case.win_len if use_w else None, sinks=sinks, rope_cs=rope_cs)


# ---- GPU calls ------------------------------------------------------------
def gpu_topk(case: Case, layer_idx: int = 0, n_visible=None, k=None, want_scores=True, ws=None):
    """ws: a workspace to (re)use; by default a fresh zeroed one."""
    cfg = case.cfg
    k = cfg.k if k is None else k
    nv = case.n_visible if n_visible is None else n_visible
    B, N = cfg.B, cfg.N
    out_idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    scores = torch.empty((B, N), dtype=torch.float32, device=DEV) if want_scores else None
    if ws is None:
        ws = torch.zeros(M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device=DEV)
    M.mla_indexer_topk(idx_row(cfg), _qi_gpu(cfg, case.inp.q_idx[layer_idx]), _t(case.inp.w[layer_idx]),
                       cfg.sigma, case.g_idx, _t(nv), k, out_idx, ws, out_scores=scores)
    torch.cuda.synchronize()
    return out_idx.cpu().numpy(), (scores.cpu().numpy() if want_scores else None)


def gpu_decode(case: Case, layer: int, idx: np.ndarray, with_window=True, sinks=None, rope_cs=None):
    cfg = case.cfg
    B, H = cfg.B, cfg.H
    k = idx.shape[1]
    out = torch.empty((B, H, cfg.d_v), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    use_w = with_window and cfg.W > 0
    win_fmt = M.MXFP8 if (use_w and case.g_win.dtype == torch.uint8) else M.BF16
    ws_n = M.mla_sparse_decode_workspace(main_row(cfg), cfg.d_v, B, H, k, cfg.W if use_w else 0, win_fmt)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=DEV)
    M.mla_sparse_decode(main_row(cfg), cfg.d_v, _q_gpu(cfg, case.inp.q[layer]), case.g_main, _t(idx),
                        cfg.softmax_scale, out, lse, ws,
                        case.g_win[layer] if use_w else None, _t(case.win_len) if use_w else None,
                        sinks=None if sinks is None else _t(np.asarray(sinks, np.float32)),
                        rope_cs=None if rope_cs is None else _t(np.asarray(rope_cs, np.float32)))
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


# ---- comparisons ----------------------------------------------------------
def check_scores(got, ref, n_visible, rel=1e-4):
    """|I_gpu - I_ref| <= rel * max(|I_ref|, rms of the visible I_ref of the row);
    masked positions must be -inf on both sides."""
    worst = 0.0
    for b in range(ref.shape[0]):
        nv = int(n_visible[b])
        r, g = ref[b, :nv].astype(np.float64), got[b, :nv].astype(np.float64)
        assert np.all(np.isneginf(got[b, nv:])) and np.all(np.isneginf(ref[b, nv:]))
        if nv == 0:
            continue
        rms = np.sqrt(np.mean(r * r))
        bound = rel * np.maximum(np.abs(r), rms)
        err = np.abs(g - r)
        worst = max(worst, float(np.max(err / np.maximum(bound, 1e-30))))
        assert np.all(err <= bound), f"row {b}: max err {err.max()} vs bound {bound[err.argmax()]}"
    return worst


def check_topk(got_idx, ref_scores, n_visible, k, rel=1e-4):
    """Set parity with the boundary exemption: positions whose oracle score lies
    within rel * max(|theta|, rms) of the oracle's k-th score theta may differ."""
    n_exempt = 0
    for b in range(got_idx.shape[0]):
        nv = int(n_visible[b])
        want = min(k, nv)
        g = got_idx[b]
        sel = g[g >= 0]
        assert np.sum(g < 0) == k - want, "wrong -1 count"
        assert len(np.unique(sel)) == len(sel), "duplicate positions"
        assert np.all(sel < nv), "masked position selected"
        if want == 0:
            continue
        r = ref_scores[b, :nv].astype(np.float64)
        order = np.lexsort((np.arange(nv), -r))
        theta = r[order[want - 1]]
        rms = np.sqrt(np.mean(r * r))
        exempt = np.abs(r - theta) <= rel * max(abs(theta), rms)
        in_ref = np.zeros(nv, bool)
        in_ref[order[:want]] = True
        in_got = np.zeros(nv, bool)
        in_got[sel] = True
        bad = (in_ref != in_got) & ~exempt
        assert not bad.any(), f"row {b}: {bad.sum()} non-exempt membership differences"
        n_exempt += int(((in_ref != in_got) & exempt).sum())
    return n_exempt


def check_attention(got_o, got_l, ref_o, ref_l, rel=2e-3):
    """Per (b, h): max_c |o - o_ref| <= rel * max_c |o_ref|; |lse - lse_ref| <= rel * max(1, |lse_ref|)."""
    B, H, _ = ref_o.shape
    worst_o = worst_l = 0.0
    for b in range(B):
        for h in range(H):
            ro, go = ref_o[b, h].astype(np.float64), got_o[b, h].astype(np.float64)
            if np.isneginf(ref_l[b, h]):
                assert np.isneginf(got_l[b, h]) and np.all(go == 0)
                continue
            scale = np.abs(ro).max()
            e = np.abs(go - ro).max()
            worst_o = max(worst_o, e / max(scale, 1e-30))
            assert e <= rel * scale, f"(b={b}, h={h}) out err {e} vs {rel * scale}"
            el = abs(float(got_l[b, h]) - float(ref_l[b, h]))
            worst_l = max(worst_l, el / max(1.0, abs(float(ref_l[b, h]))))
            assert el <= rel * max(1.0, abs(float(ref_l[b, h]))), f"(b={b}, h={h}) lse err {el}"
    return worst_o, worst_l
