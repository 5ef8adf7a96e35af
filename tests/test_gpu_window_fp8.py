"""MXFP8 window entries (E4M3 codes with one E8M0 scale per 32 channels: V4.1's
528-byte window entry, [P1] "DeepSeek-V4.1"): the append writes the oracle's
bytes exactly, and the decode over such a ring matches the oracle's attention
over the dequantised entries (which are exact in bf16 for these inputs)."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
import sparse_latent_attention_mla_amd as M
import workloads as WL
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu


def _window_values(B, W, D, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((W, B, D)) * np.exp2(rng.integers(-12, 12, (W, B, 1)))
    v[0, 0, :32] = 0.0                                  # a block of zeros
    v[1, 0, 5] = -0.0
    v[2, 0, 32:64] *= np.exp2(np.arange(32) - 16)      # a wide block: subnormal E4M3 codes
    v[3, 0, 64] = 1e6                                  # one dominant value per block
    v[4, 0, 96:128] = 447.9                            # near the top of the E4M3 range
    return v.astype(np.float32)


C = WL.CONFIGS
SMALL = {                                              # (V3.2's shapes given a window: 576-channel entries)
    "c3w": C["c3"].with_(name="c3w", cid=123, B=2, N=6001, W=64),
    "c4s": C["c4"].with_(name="c4s", cid=104, B=2, N=4099),
    "c5s": C["c5"].with_(name="c5s", cid=105, B=1, N=3001),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_mxfp8_window_append_bytes_and_decode(name):
    cfg = SMALL[name]
    if cfg.W == 0:
        pytest.skip("no window in this configuration")
    print("mxfp8 window", name, flush=True)
    case = G.build_case(cfg, seed=3)
    B, W, D = cfg.B, cfg.W, cfg.dim + cfg.rope
    vals = _window_values(B, W, D, cfg.cid + 31)
    ring = torch.zeros((B, W, D + D // 32), dtype=torch.uint8, device=G.DEV)
    mr, ir = G.main_row(cfg), G.idx_row(cfg)
    for i in range(W):                                  # slot i <- window entry i
        M.mla_kv_append_quant(mr, ir, None, None, None, None, None, G._t(vals[i]),
                              G._t(np.full(B, i, np.int32)), ring)
    torch.cuda.synchronize()
    want = O.quant_rows(O.MXFP8, D, 0, vals.transpose(1, 0, 2).reshape(-1, D)).reshape(B, W, -1)
    got = ring.cpu().numpy()
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:4].tolist()}"
    # the oracle's attention over the dequantised entries, carried as bf16 (exact here)
    deq = O.dequant_rows(O.MXFP8, D, 0, want.reshape(-1, D + D // 32))
    as_bf16 = torch.from_numpy(deq.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(as_bf16.float().numpy().astype(np.float64), deq)
    o_win = as_bf16.view(torch.int16).numpy().view(np.uint16).reshape(1, B, W, D)
    case8 = dataclasses.replace(case, o_win=o_win, g_win=ring.unsqueeze(0))
    rng = np.random.default_rng(cfg.cid + 37)            # any selection will do: distinct visible rows, some -1
    idx = np.stack([rng.permutation(int(n))[:cfg.k] for n in case8.n_visible]).astype(np.int32)
    idx[:, ::7] = -1
    ref_o, ref_l = G.oracle_attention(case8, 0, idx)
    got_o, got_l = G.gpu_decode(case8, 0, idx)
    launched = M.mla_last_kernels()
    # 512-channel entries are widened as the decode stages them; 576-channel ones (594 bytes,
    # not 16-byte aligned) by a widening launch first
    assert any("k_widen_window" in k for k in launched) == (D != 512), launched
    G.check_attention(got_o, got_l, ref_o, ref_l)
    # the same entries as a bf16 ring give the same decode up to summation order
    case16 = dataclasses.replace(case, o_win=o_win, g_win=as_bf16.reshape(1, B, W, D).to(G.DEV))
    got16_o, got16_l = G.gpu_decode(case16, 0, idx)
    np.testing.assert_allclose(got_o, got16_o, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(got_l, got16_l, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("name", ["c3w", "c4s"])
def test_mxfp8_window_in_the_carried_append(name):
    """mla_append_indexer_topk with an MXFP8 ring: the window entry rides in the
    scan's launch (one wave per 128-channel slice) and its bytes equal the oracle's."""
    cfg = SMALL[name]
    print("mxfp8 carried window", name, flush=True)
    B, N, D, k = cfg.B, cfg.N, cfg.dim + cfg.rope, cfg.k
    rng = np.random.default_rng(cfg.cid + 41)
    mr, ir = G.main_row(cfg), G.idx_row(cfg)
    main = torch.zeros((B, N, M.row_bytes(mr)), dtype=torch.uint8, device=G.DEV)
    idx_c = torch.zeros((B, N, M.row_bytes(ir)), dtype=torch.uint8, device=G.DEV)
    ring = torch.zeros((B, cfg.W, D + D // 32), dtype=torch.uint8, device=G.DEV)
    vals = _window_values(B, 5, D, cfg.cid + 43)[2]         # entry 2: a wide block in sequence 0
    vals[-1, :32] = 0.0                                    # and a block of zeros
    pos = np.array([5 + 3 * b for b in range(B)], np.int32)
    new_main = G._t(rng.standard_normal((B, 1, D)).astype(np.float32))
    new_idx = G._t(rng.standard_normal((B, 1, cfg.d_I)).astype(np.float32))
    slots = G._t(np.full((B, 1), N - 1, np.int32))
    qi = G._qi_gpu(cfg, rng.standard_normal((B, cfg.H_I, cfg.d_I)).astype(np.float32))
    w = G._t(rng.standard_normal((B, cfg.H_I)).astype(np.float32))
    out_idx = torch.empty((B, k), dtype=torch.int32, device=G.DEV)
    ws = torch.zeros(M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device=G.DEV)
    M.mla_append_indexer_topk(mr, ir, new_main, new_idx, slots, main, idx_c, qi, w, cfg.sigma,
                              G._t(np.full(B, N, np.int32)), k, out_idx, ws,
                              new_win=G._t(vals), win_pos=G._t(pos), win_ring=ring)
    torch.cuda.synchronize()
    want = O.quant_rows(O.MXFP8, D, 0, vals)
    got = ring.cpu().numpy()
    for b in range(B):
        assert np.array_equal(got[b, pos[b] % cfg.W], want[b]), f"sequence {b}"
        others = np.delete(got[b], pos[b] % cfg.W, axis=0)
        assert not others.any(), "only the entry's slot is written"
