"""mla_append_sparse_decode: the step's window entry appended to the ring, then the
decode, in one call ([P1] "DeepSeek-V4", "A window in every layer"; "DeepSeek-V4.1",
"Three modes": a Reuse layer's step). The ring must end up holding the oracle's bytes
of the entry in slot win_pos mod W (no change for win_pos < 0), and the decode must
match the oracle's attention over that ring. 512-channel bf16 and MXFP8 entries are
written by the decode's own window split (no other launch); the 576-channel entry
takes an append launch first. The target slots are poisoned beforehand."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import workloads as WL
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
C = WL.CONFIGS
CASES = {
    "c4t": C["c4"].with_(name="c4t", cid=161, B=3, N=3001),                       # E2M1 rows, 512-ch window
    "c2w": C["c2"].with_(name="c2w", cid=162, B=1, N=2100, rope=0, W=96, softmax_scale=512 ** -0.5),  # bf16 rows
    "c3w": C["c3"].with_(name="c3w", cid=163, B=2, N=2500, W=64),                 # 576-ch window: append launch
}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


@pytest.mark.parametrize("win_fmt", ["bf16", "mxfp8"])
@pytest.mark.parametrize("name", sorted(CASES))
def test_append_then_decode_in_one_call(name, win_fmt):
    cfg = CASES[name]
    print("window append + decode", name, win_fmt, flush=True)
    case = G.build_case(cfg, seed=2)
    M = G.M
    B, W, D = cfg.B, cfg.W, cfg.dim + cfg.rope
    p = cfg.tokens - 1
    rng = np.random.default_rng(cfg.cid)
    new = rng.standard_normal((B, D)).astype(np.float32) * np.float32(3.0)
    # own slot, another slot (past sequence 1's window length: written, not attended), none
    pos = {1: [p - 5], 2: [p - 5, -1], 3: [p, p - 5, -1]}[B]
    pos = np.array(pos, np.int32)
    # the ring before the call (the case's window values), on both sides
    if win_fmt == "bf16":
        ring_o = case.o_win[0].copy()                            # uint16 bf16 [B, W, D]
        ring_g = case.g_win[0].clone()
        want = ring_o.copy()
        for b in range(B):
            if pos[b] >= 0:
                want[b, pos[b] % W] = O.bf16_encode(new[b]).astype(np.uint16)
        want_bytes = want.view(np.uint8)
        deq = O.bf16_value(want.reshape(-1)).reshape(B, W, D).astype(np.float64)
    else:
        vals = O.bf16_value(case.o_win[0].reshape(-1)).reshape(B, W, D).astype(np.float32)
        ring_o = O.quant_rows(O.MXFP8, D, 0, vals.reshape(-1, D)).reshape(B, W, -1)
        ring_g = torch.from_numpy(ring_o.copy()).to(G.DEV)
        want = ring_o.copy()
        for b in range(B):
            if pos[b] >= 0:
                want[b, pos[b] % W] = O.quant_rows(O.MXFP8, D, 0, new[b:b + 1])[0]
        want_bytes = want
        deq = O.dequant_rows(O.MXFP8, D, 0, want.reshape(-1, D + D // 32)).reshape(B, W, D)
    for b in range(B):                                           # poison the slots the call must write
        if pos[b] >= 0:
            ring_g.view(torch.uint8)[b, pos[b] % W] = 0x5A
    as_bf16 = torch.from_numpy(deq.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(as_bf16.float().numpy().astype(np.float64), deq)   # exact in bf16 (the oracle's view)
    o_win = as_bf16.view(torch.int16).numpy().view(np.uint16).reshape(1, B, W, D)
    win_len = np.array([W, (p - 5) % W, 1][:B], np.int32)
    ref_case = dataclasses.replace(case, o_win=o_win, win_len=win_len)
    idx = np.stack([rng.permutation(cfg.N)[:cfg.k] for _ in range(B)]).astype(np.int32)
    idx[:, ::5] = -1
    ref_o, ref_l = G.oracle_attention(ref_case, 0, idx)

    out = torch.empty((B, cfg.H, cfg.d_v), dtype=torch.float32, device=G.DEV)
    lse = torch.empty((B, cfg.H), dtype=torch.float32, device=G.DEV)
    wfmt = M.MXFP8 if win_fmt == "mxfp8" else M.BF16
    ws = torch.empty(max(1, M.mla_sparse_decode_workspace(G.main_row(cfg), cfg.d_v, B, cfg.H, cfg.k, W, wfmt)),
                     dtype=torch.uint8, device=G.DEV)
    M.mla_sparse_decode(G.main_row(cfg), cfg.d_v, G._q_gpu(cfg, case.inp.q[0]), case.g_main, G._t(idx),
                        cfg.softmax_scale, out, lse, ws, ring_g, G._t(win_len), new_win=G._t(new), win_pos=G._t(pos))
    launched = M.mla_last_kernels()
    torch.cuda.synchronize()
    fused = D == 512
    assert any("k_append" in k for k in launched) != fused, launched
    got = ring_g.view(torch.uint8).cpu().numpy()
    bad = np.argwhere(got != want_bytes)
    assert bad.size == 0, f"{len(bad)} ring bytes differ, first at {bad[:4].tolist()}"
    G.check_attention(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l)
