"""Quantisation on the GPU lands on the oracle's codes exactly where the tie
rule decides ([P1] "A Precision Primer", "FP8: E4M3 and E5M2" and "E2M1: eight
magnitudes"): inputs built to sit on midpoints between codes (and one fp32 step
beside them), block maxima whose E4M3 scale is itself rounded from a midpoint,
zero and saturating scales, in every row format, through the three calls that
quantise: mla_kv_append_quant, the append carried by mla_append_indexer_topk,
and mla_compress_append. Byte-exact against the oracle. A sweep over every
16th fp32 bit pattern up to 448 at unit block scale checks the E4M3 encoder
against the oracle's on 71 million values, and a sweep of FP4 block maxima the
E4M3 rounding of amax / 6."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_latent_attention_mla_amd as M
from tests import codec_rows as R

pytestmark = pytest.mark.gpu
DEV = "cuda"
FM = {"E4M3_S128": O.E4M3_S128, "E2M1_S16": O.E2M1_S16, "MXFP4": O.MXFP4, "MXFP8": O.MXFP8, "BF16": O.BF16}
# (main row, indexer row): the configurations' pairs
PAIRS = {
    "v32_e4m3": ((O.E4M3_S128, 512, 64), (O.E4M3_S128, 128, 0)),
    "v41_e2m1": ((O.E2M1_S16, 512, 0), (O.E2M1_S16, 128, 0)),
    "v41_mxfp4_keys": ((O.E2M1_S16, 512, 0), (O.MXFP4, 128, 0)),
}


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def _rows(rng, row, n):
    """n rows: half grid rows (where the format has them), half ulp rows."""
    fmt, dim, rope = row
    out = []
    for i in range(n):
        if i % 2 == 0 and fmt in (O.E4M3_S128, O.E2M1_S16, O.MXFP4):
            out.append(R.grid_row(rng, fmt, dim, rope, FM))
        else:
            out.append(R.ulp_row(rng, fmt, dim, rope, FM))
    return np.stack(out).astype(np.float32)


def _win_rows(rng, fmt, D, n):
    return np.stack([R.ulp_row(rng, fmt, D, 0, FM) for _ in range(n)]).astype(np.float32)


@pytest.mark.parametrize("pair", sorted(PAIRS))
def test_append_midpoints(pair):
    mr, ir = PAIRS[pair]
    print("append midpoints", pair, flush=True)
    rng = np.random.default_rng(100 + len(pair))
    B, n = 4, 64
    main = _rows(rng, mr, B * n).reshape(B, n, -1)
    idx = _rows(rng, ir, B * n).reshape(B, n, -1)
    slots = np.tile(np.arange(n, dtype=np.int32), (B, 1))
    rb, rbi = O.row_bytes(*mr), O.row_bytes(*ir)
    o_main = np.zeros((B, n, rb), np.uint8)
    o_idx = np.zeros((B, n, rbi), np.uint8)
    O.append(mr, ir, main, idx, slots, o_main, o_idx)
    g_main = torch.zeros((B, n, rb), dtype=torch.uint8, device=DEV)
    g_idx = torch.zeros((B, n, rbi), dtype=torch.uint8, device=DEV)
    M.mla_kv_append_quant(M.Row(*mr), M.Row(*ir), _t(main), _t(idx), _t(slots), g_main, g_idx)
    torch.cuda.synchronize()
    assert np.array_equal(g_main.cpu().numpy(), o_main), "main rows differ"
    assert np.array_equal(g_idx.cpu().numpy(), o_idx), "indexer rows differ"


@pytest.mark.parametrize("wfmt", ["bf16", "mxfp8"])
def test_window_append_midpoints(wfmt):
    print("window midpoints", wfmt, flush=True)
    rng = np.random.default_rng(7 if wfmt == "bf16" else 8)
    B, W, D = 4, 32, 512
    fmt = O.BF16 if wfmt == "bf16" else O.MXFP8
    ent = _win_rows(rng, fmt, D, B * W).reshape(B, W, D)
    if wfmt == "bf16":
        ring = torch.zeros((B, W, D), dtype=torch.bfloat16, device=DEV)
    else:
        ring = torch.zeros((B, W, D + D // 32), dtype=torch.uint8, device=DEV)
    r0 = M.Row(O.E4M3_S128, 128, 0)
    for s in range(W):
        M.mla_kv_append_quant(r0, r0, None, None, None, None, None, _t(ent[:, s]),
                              _t(np.full(B, s, np.int32)), ring)
    torch.cuda.synchronize()
    if wfmt == "bf16":
        got = ring.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, O.bf16_encode(ent))
    else:
        assert np.array_equal(ring.cpu().numpy(), O.quant_rows(O.MXFP8, D, 0, ent))


# MXFP8 window entries of 512 channels go with the 512-channel (V4.1) rows
FUSED = [(p, w) for p in sorted(PAIRS) for w in ("bf16", "mxfp8", None)
         if not (w == "mxfp8" and sum(PAIRS[p][0][1:]) != 512)]


@pytest.mark.parametrize("pair,wfmt", FUSED)
def test_fused_append_midpoints(pair, wfmt):
    """The append carried in the LDS-DMA scan's launch (16-byte aligned sequence
    ends): four entries per sequence and the window entry, in eight calls, against
    the oracle."""
    mr, ir = PAIRS[pair]
    D = mr[1] + mr[2]
    print("fused append midpoints", pair, wfmt, flush=True)
    rng = np.random.default_rng(200 + len(pair) + (0 if wfmt is None else len(wfmt)))
    B, N, n, H_I, k, W = 4, 16388, 4, 64, 64, 128
    rb, rbi = O.row_bytes(*mr), O.row_bytes(*ir)
    g_main = torch.zeros((B, N, rb), dtype=torch.uint8, device=DEV)
    g_idx = torch.zeros((B, N, rbi), dtype=torch.uint8, device=DEV)
    q_idx = torch.from_numpy(rng.standard_normal((B, H_I, ir[1])).astype(np.float32)).to(torch.bfloat16).to(DEV)
    w = _t((rng.standard_normal((B, H_I)) * 0.125).astype(np.float32))
    nv = _t(np.full(B, N, np.int32))
    out = torch.empty((B, k), dtype=torch.int32, device=DEV)
    ws = torch.zeros(M.mla_indexer_topk_workspace(B, N, k), dtype=torch.uint8, device=DEV)
    ring = None
    if wfmt:
        ring = (torch.zeros((B, W, D), dtype=torch.bfloat16, device=DEV) if wfmt == "bf16" else
                torch.zeros((B, W, D + D // 32), dtype=torch.uint8, device=DEV))
    for rep in range(8):
        main = _rows(rng, mr, B * n).reshape(B, n, -1)
        idx = _rows(rng, ir, B * n).reshape(B, n, -1)
        slots = np.stack([np.sort(rng.choice(N, n, replace=False)) for _ in range(B)]).astype(np.int32)
        win = {}
        if wfmt:
            ent = _win_rows(rng, O.BF16 if wfmt == "bf16" else O.MXFP8, D, B)
            pos = rng.integers(0, 10 ** 6, B).astype(np.int32)
            win = dict(new_win=_t(ent), win_pos=_t(pos), win_ring=ring)
        M.mla_append_indexer_topk(M.Row(*mr), M.Row(*ir), _t(main), _t(idx), _t(slots), g_main, g_idx, q_idx, w,
                                  0.088, nv, k, out, ws, **win)
        launched = M.mla_last_kernels()
        torch.cuda.synchronize()
        scans = [x for x in launched if "k_scan" in x or "k_append" in x]
        assert len(scans) == 1 and "k_scan_dma32" in scans[0] and "true>(" in scans[0], launched
        o_main = np.zeros((B, n, rb), np.uint8)
        o_idx = np.zeros((B, n, rbi), np.uint8)
        O.append(mr, ir, main, idx, np.tile(np.arange(n, dtype=np.int32), (B, 1)), o_main, o_idx)
        gm = g_main.cpu().numpy()[np.arange(B)[:, None], slots]
        gi = g_idx.cpu().numpy()[np.arange(B)[:, None], slots]
        assert np.array_equal(gm, o_main), f"call {rep}: main rows differ"
        assert np.array_equal(gi, o_idx), f"call {rep}: indexer rows differ"
        if wfmt:
            sl = pos % W
            if wfmt == "bf16":
                got = ring.cpu().view(torch.int16).numpy().view(np.uint16)[np.arange(B), sl]
                assert np.array_equal(got, O.bf16_encode(ent)), f"call {rep}: window entries differ"
            else:
                got = ring.cpu().numpy()[np.arange(B), sl]
                assert np.array_equal(got, O.quant_rows(O.MXFP8, 512, 0, ent)), f"call {rep}: window entries differ"


@pytest.mark.parametrize("row", [(O.E4M3_S128, 512, 64), (O.E2M1_S16, 512, 0), (O.MXFP4, 128, 0)])
def test_compress_midpoints(row):
    """A one-token window with unit norm weight and eps 0 returns the grid row
    itself (mean square exactly 1); its quantised row then meets the midpoints."""
    fmt, dim, rope = row
    print("compress midpoints", row, flush=True)
    rng = np.random.default_rng(300 + fmt)
    B = 48
    kv = np.stack([R.grid_row(rng, fmt, dim, rope, FM) for _ in range(B)])[:, None, :]
    gate = rng.standard_normal(kv.shape).astype(np.float32)
    cache = torch.zeros((B, 2, O.row_bytes(*row)), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, dim + rope), dtype=torch.float32, device=DEV)
    M.mla_compress_append(M.Row(*row), _t(kv), _t(gate), cache, _t(np.ones(B, np.int32)), None, 0.0,
                          out_entry=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, kv[:, 0]), "the entry is not the row"
    assert np.array_equal(cache.cpu().numpy()[:, 1], O.quant_rows(fmt, dim, rope, kv[:, 0]))
    assert not cache.cpu().numpy()[:, 0].any()


def test_e4m3_sweep_at_unit_scale():
    """Every 16th fp32 bit pattern from the smallest subnormal up to 448 (and
    their negatives), 127 per 128-channel block beside a 448 (scale exactly 1):
    the GPU's codes equal the oracle's E4M3 encoder's."""
    print("e4m3 sweep", flush=True)
    bits = np.arange(1, 0x43E00001, 16, dtype=np.uint32)
    vals = bits.view(np.float32)
    vals = np.concatenate([vals, -vals])
    n_rows = -(-vals.size // 127)
    x = np.zeros((n_rows, 128), np.float32)
    x[:, 0] = 448.0
    flat = x[:, 1:].reshape(-1)
    flat[:vals.size] = vals
    x[:, 1:] = flat.reshape(n_rows, 127)
    want = O.e4m3_encode(x[:, 1:])
    row = M.Row(O.E4M3_S128, 128, 0)
    chunk = 1 << 18
    for r0 in range(0, n_rows, chunk):
        xr = x[r0:r0 + chunk]
        n = xr.shape[0]
        cache = torch.zeros((1, n, 132), dtype=torch.uint8, device=DEV)
        M.mla_kv_append_quant(row, row, None, _t(xr[None]), _t(np.arange(n, dtype=np.int32)[None]), None, cache)
        got = cache.cpu().numpy()[0]
        assert np.all(got[:, 128:132].view(np.float32) == 1.0)
        bad = np.flatnonzero(np.any(got[:, 1:128] != want[r0:r0 + n], axis=1))
        assert bad.size == 0, f"rows {r0 + bad[:4]} differ"


def test_fp4_scale_sweep():
    """FP4 block maxima over 2^20 fp32 bit patterns spanning the E4M3 scale range
    (amax / 6 from below half the smallest subnormal to past 448): the E4M3 scale
    byte and the codes equal the oracle's."""
    print("fp4 scale sweep", flush=True)
    lo, hi = np.float32(6 * 2.0 ** -12).view(np.uint32), np.float32(6 * 600.0).view(np.uint32)
    amax = np.linspace(lo, hi, 1 << 20).astype(np.uint32).view(np.float32)
    rng = np.random.default_rng(9)
    x = (rng.uniform(-1, 1, (amax.size, 16)) * amax[:, None]).astype(np.float32)
    x[:, 0] = amax
    x = x.reshape(-1, 512)
    row = M.Row(O.E2M1_S16, 512, 0)
    cache = torch.zeros((1, x.shape[0], 288), dtype=torch.uint8, device=DEV)
    M.mla_kv_append_quant(row, row, _t(x[None]), None, _t(np.arange(x.shape[0], dtype=np.int32)[None]), cache, None)
    got = cache.cpu().numpy()[0]
    want = O.quant_rows(O.E2M1_S16, 512, 0, x)
    bad = np.flatnonzero(np.any(got != want, axis=1))
    assert bad.size == 0, f"rows {bad[:4]} differ"
