"""Pins of the oracle's formats and codecs to things outside the oracle:
library casts, the pages' printed worked example and byte counts, closed forms.
CPU only."""
import json
import os

import numpy as np
import pytest
import torch

import oracle as O

E2M1_LADDER = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


# ---- E4M3 ----------------------------------------------------------------
def test_e4m3_decode_matches_library_fp8_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = O.e4m3_value(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert nan.sum() == 2                       # one NaN pattern per sign
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_closed_form_facts():
    v = O.e4m3_value(np.arange(128))
    fin = v[~np.isnan(v)]
    pos = fin[fin > 0]
    assert pos.max() == 448.0                   # largest finite value
    assert len(pos) == 126                      # positive finite non-zero codes
    binades = np.unique(np.floor(np.log2(pos)))
    assert len(binades) == 18                   # "from 17 to 18 binades"
    assert binades.min() == -9 and binades.max() == 8


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.e4m3_value(codes).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), codes)


def test_e4m3_encode_matches_library_rne_cast():
    rng = np.random.default_rng(1)
    grid = O.e4m3_value(np.arange(0x7F)).astype(np.float64)        # 0 .. 448
    mids = (grid[:-1] + grid[1:]) / 2                               # exact ties
    x = np.concatenate([
        rng.standard_normal(20000) * 30,
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 1e-2,
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
        [0.0, -0.0, 448.0, -448.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 1e-30],
    ]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x), ref)


def test_e4m3_encode_saturates_beyond_448():
    x = np.array([448.0, 449.0, 464.0, 470.0, 1e6, -500.0, -1e30], dtype=np.float32)
    assert list(O.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]


# ---- E2M1 ----------------------------------------------------------------
def test_e2m1_values_are_the_pages_eight_magnitudes():
    assert list(O.e2m1_value(np.arange(8))) == E2M1_LADDER
    assert list(O.e2m1_value(np.arange(8, 16))) == [-v for v in E2M1_LADDER]


def _nearest_rung_brute_force(y):
    """Exhaustive search over the 16 codes: nearest value, ties to the code
    with an even mantissa bit, saturating beyond +-6 by nearness."""
    vals = np.array(E2M1_LADDER)
    out = []
    for t in y:
        a = abs(float(t))
        dist = np.abs(vals - a)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:                      # a tie between two rungs
            best = [b for b in best if (b & 1) == 0]
        code = int(best[0])
        out.append(code | (8 if np.signbit(t) else 0))
    return np.array(out, dtype=np.uint8)


def test_e2m1_encode_matches_brute_force_nearest_rung():
    rng = np.random.default_rng(2)
    ladder = np.array(E2M1_LADDER)
    mids = (ladder[:-1] + ladder[1:]) / 2
    y = np.concatenate([rng.uniform(-7, 7, 20000), rng.standard_normal(5000) * 0.3,
                        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 10),
                        ladder, -ladder, [6.5, -6.5, 100.0, -1e9, 7.0]]).astype(np.float32)
    assert np.array_equal(O.e2m1_encode(y), _nearest_rung_brute_force(y))


# ---- bf16 ----------------------------------------------------------------
def test_bf16_encode_matches_library_cast():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(50000), rng.standard_normal(20000) * 1e30,
                        rng.standard_normal(20000) * 1e-30]).astype(np.float32)
    # exact ties: low half == 0x8000 with both parities of the kept part
    u = rng.integers(0, 2 ** 31, 4000, dtype=np.uint32) & np.uint32(0x7F7F0000)
    ties = (u | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties, -ties, [0.0, -0.0, np.float32(3.4e38)]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.bf16_encode(x), ref)


# ---- rows ----------------------------------------------------------------
def test_row_sizes_match_the_pages(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kv_bytes.json")))
    assert O.row_bytes(O.E4M3_S128, 512, 64) == g["v32"]["main_row"] == 656
    assert O.row_bytes(O.E4M3_S128, 128, 0) == g["v32"]["indexer_row"] == 132
    assert g["v32"]["layers"] * (656 + 132) == g["v32"]["bytes_per_token"]
    assert O.row_bytes(O.E2M1_S16, 512, 0) == g["v41"]["main_row"] == 288
    assert O.row_bytes(O.E2M1_S16, 128, 0) == g["v41"]["indexer_row_same_format"] == 72
    v41 = g["v41"]
    assert v41["entries_per_token"] * (288 + v41["indexer_row_mxfp4"]) == v41["bytes_per_token_published"]
    assert v41["entries_per_token"] * (288 + 72) == v41["bytes_per_token_with_72"]
    assert abs(900 - 890) / 890 < 0.012                              # "within about one per cent"
    assert O.row_bytes(O.BF16, 512, 64) == 1152 and O.row_bytes(O.BF16, 128, 0) == 256
    assert O.row_bytes(O.F32, 64, 16) == 320 and O.row_bytes(O.F32, 32, 0) == 128
    # the MXFP4 indexer key: 128 nibbles + four E8M0 scales, the 68 B the pages' total needs
    assert O.row_bytes(O.MXFP4, 128, 0) == v41["indexer_row_mxfp4"] == 68
    assert v41["entries_per_token"] * (288 + O.row_bytes(O.MXFP4, 128, 0)) == 890
    # unsupported shapes are refused
    assert O.row_bytes(O.E4M3_S128, 100, 0) < 0 and O.row_bytes(O.E2M1_S16, 512, 64) < 0
    assert O.row_bytes(O.MXFP4, 48, 0) < 0 and O.row_bytes(O.MXFP4, 128, 2) < 0


def test_fp4_row_reproduces_the_pages_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "fp4_worked_example.json")))
    rng = np.random.default_rng(0)
    latent = rng.standard_normal(512)
    latent *= np.sqrt(512) / np.linalg.norm(latent)
    x = latent.astype(np.float32)
    rows = O.quant_rows(O.E2M1_S16, 512, 0, x[None])
    assert rows.shape[-1] == g["printed"]["bytes_per_512ch_entry"]["fp4_e4m3_16"]
    deq = O.dequant_rows(O.E2M1_S16, 512, 0, rows)[0]
    rel = np.linalg.norm(deq - x) / np.linalg.norm(x)
    assert round(float(np.abs(x).max()), 3) == g["printed"]["max_abs_latent"]
    assert round(float(rel), 4) == g["printed"]["rel_l2_error"]


def test_fp4_row_error_bound_and_scale_rule():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, 512)) * rng.uniform(0.01, 50, (64, 1))).astype(np.float32)
    rows = O.quant_rows(O.E2M1_S16, 512, 0, x)
    deq = O.dequant_rows(O.E2M1_S16, 512, 0, rows)
    sc = O.e4m3_value(rows[:, 256:]).astype(np.float64)          # [64, 32] block scales
    amax = np.abs(x.reshape(64, 32, 16)).max(-1)
    # the scale is the E4M3 rounding of amax / 6
    assert np.array_equal(rows[:, 256:], O.e4m3_encode((amax / np.float32(6)).astype(np.float32)))
    s = np.repeat(sc, 16, axis=1)
    y = x / s
    unclipped = np.abs(y) <= 6
    # nearest rung: the largest gap of the ladder is 2, so the error is at most one scale unit
    assert np.all(np.abs(deq - x)[unclipped] <= s[unclipped] * (1 + 1e-6))
    # the dequantised value is an exact product of a rung and the scale
    assert np.all(np.isin(np.abs(deq / s), E2M1_LADDER))


def test_fp4_nibble_order_and_zero_block():
    x = np.zeros(512, np.float32)
    x[:16] = [6, 0.5, 1, 1.5, 2, 3, 4, -6, -0.5, 0, 0, 0, 0, 0, 0, 0]   # scale E4M3(1.0)
    r = O.quant_rows(O.E2M1_S16, 512, 0, x[None])[0]
    assert r[256] == 0x38                                          # E4M3 code of 1.0
    assert r[0] == (0x7 | (0x1 << 4)) and r[3] == (0xF << 4 | 0x6)  # low nibble = even channel
    assert np.all(r[8:256] == 0) and np.all(r[257:] == 0)           # all-zero blocks: scale 0, codes 0


def test_fp8_row_layout_error_bound_and_rope_tail():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((32, 576)) * rng.uniform(0.001, 100, (32, 1))).astype(np.float32)
    rows = O.quant_rows(O.E4M3_S128, 512, 64, x)
    assert rows.shape[-1] == 656
    deq = O.dequant_rows(O.E4M3_S128, 512, 64, rows)
    scales = rows[:, 512:528].copy().view(np.float32)              # four fp32 scales
    amax = np.abs(x[:, :512].reshape(32, 4, 128)).max(-1)
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    lat, dl = x[:, :512].astype(np.float64), deq[:, :512]
    s = np.repeat(scales.astype(np.float64), 128, axis=1)
    normal = np.abs(lat / s) >= 2.0 ** -6
    assert np.all(np.abs(dl - lat)[normal] <= 2.0 ** -4 * np.abs(lat)[normal] * (1 + 1e-6))
    assert np.all(np.abs(dl - lat)[~normal] <= 2.0 ** -10 * s[~normal] * (1 + 1e-6))
    # rope tail: bf16 of the input
    tail = rows[:, 528:].copy().view(np.uint16)
    ref = torch.from_numpy(x[:, 512:].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(tail, ref)
    # the block maximum decodes back to itself up to the fp32 rounding of the scale
    i = np.abs(lat.reshape(32, 4, 128)).argmax(-1)
    got = np.take_along_axis(np.abs(dl.reshape(32, 4, 128)), i[..., None], -1)[..., 0]
    assert np.allclose(got, amax, rtol=2.0 ** -22, atol=0)


def test_bf16_and_f32_rows():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 80)).astype(np.float32)
    assert np.array_equal(O.dequant_rows(O.F32, 64, 16, O.quant_rows(O.F32, 64, 16, x)), x)
    r = O.quant_rows(O.BF16, 512, 64, np.resize(x, (8, 576)))
    ref = torch.from_numpy(np.resize(x, (8, 576))).to(torch.bfloat16).float().numpy()
    assert np.array_equal(O.dequant_rows(O.BF16, 512, 64, r), ref)


def test_append_writes_only_its_slots_and_the_window_ring():
    rng = np.random.default_rng(7)
    B, cap, W = 3, 40, 8
    main = np.full((B, cap, 288), 0xAB, np.uint8)
    idx = np.full((B, cap, 72), 0xCD, np.uint8)
    ring = np.zeros((B, W, 512), np.uint16)
    new_main = rng.standard_normal((B, 2, 512)).astype(np.float32)
    new_idx = rng.standard_normal((B, 2, 128)).astype(np.float32)
    slots = np.array([[3, 4], [0, 39], [17, 18]], np.int32)
    new_win = rng.standard_normal((B, 512)).astype(np.float32)
    pos = np.array([5, 8, 100], np.int32)
    O.append((O.E2M1_S16, 512, 0), (O.E2M1_S16, 128, 0), new_main, new_idx, slots,
             main, idx, new_win, pos, ring)
    for b in range(B):
        for i in range(2):
            s = slots[b, i]
            assert np.array_equal(main[b, s], O.quant_rows(O.E2M1_S16, 512, 0, new_main[b, i][None])[0])
            assert np.array_equal(idx[b, s], O.quant_rows(O.E2M1_S16, 128, 0, new_idx[b, i][None])[0])
        untouched = np.setdiff1d(np.arange(cap), slots[b])
        assert np.all(main[b, untouched] == 0xAB) and np.all(idx[b, untouched] == 0xCD)
        assert np.array_equal(ring[b, pos[b] % W], O.bf16_encode(new_win[b]))
        others = [j for j in range(W) if j != pos[b] % W]
        assert np.all(ring[b, others] == 0)
    with pytest.raises(ValueError):
        O.append((O.E2M1_S16, 512, 0), (O.E2M1_S16, 128, 0), new_main, new_idx,
                 np.array([[0, 40]] * 3, np.int32), main, idx)


# ---- MXFP4 (E2M1 elements, one E8M0 power-of-two scale per 32 channels) ----
def test_e8m0_values_and_the_mx_scale_rule():
    assert list(O.e8m0_value([127, 128, 126, 0, 254])) == [1.0, 2.0, 0.5, 2.0 ** -127, 2.0 ** 127]
    assert np.isnan(O.e8m0_value([255])[0])
    # X = 2^(floor(log2 amax) - 2): the block maximum lands in [4, 8) scale units
    assert O.mx_scale(6.0) == 127 and O.mx_scale(4.0) == 127 and O.mx_scale(7.99) == 127
    assert O.mx_scale(1.0) == 125 and O.mx_scale(3.99) == 126 and O.mx_scale(8.0) == 128
    assert O.mx_scale(0.0) == 0 and O.mx_scale(2.0 ** -140) == 0          # clamped at the smallest code
    assert O.mx_scale(3.0e38) == 127 + 127 - 2                           # floor(log2 3e38) = 127
    rng = np.random.default_rng(11)
    a = (rng.uniform(0.5, 1.0, 500) * 2.0 ** rng.integers(-60, 60, 500)).astype(np.float32)
    X = O.e8m0_value([O.mx_scale(v) for v in a])
    assert np.all((a / X >= 4) & (a / X < 8))


def test_mxfp4_row_roundtrip_error_bound_and_layout():
    rng = np.random.default_rng(12)
    # blocks on the grid (a rung of 4 or 6 present, so the block maximum picks the scale) round-trip
    nib = rng.integers(0, 16, (40, 128)).astype(np.uint32)
    nib[:, ::32] = rng.choice([0x6, 0x7, 0xE, 0xF], (40, 4))              # +-4 or +-6 in every block
    e = rng.integers(100, 150, (40, 4))
    x = (O.e2m1_value(nib) * np.repeat(2.0 ** (e - 127), 32, axis=1)).astype(np.float32)
    r = O.quant_rows(O.MXFP4, 128, 0, x)
    assert np.array_equal(O.dequant_rows(O.MXFP4, 128, 0, r), x)
    assert np.array_equal(r[:, 64:], e.astype(np.uint8))
    # low nibble = even channel
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    assert np.array_equal(r[:, :64], packed)
    # general inputs: nearest rung below 6X (largest gap 2X), saturation above
    y = (rng.standard_normal((64, 128)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    ry = O.quant_rows(O.MXFP4, 128, 0, y)
    d = O.dequant_rows(O.MXFP4, 128, 0, ry)
    Xs = np.repeat(O.e8m0_value(ry[:, 64:]), 32, axis=1)
    small = np.abs(y) <= 6 * Xs
    assert np.all(np.abs(d - y)[small] <= Xs[small])
    assert np.all(np.abs(d[~small]) == 6 * Xs[~small])
    assert np.all(np.isin(np.abs(d / Xs), E2M1_LADDER))
    # a block of zeros: scale code 0, codes 0
    z = np.zeros((1, 128), np.float32)
    assert not O.quant_rows(O.MXFP4, 128, 0, z).any()


def test_mxfp8_window_entry_size_scale_rule_and_hand_encoded_codes():
    # the V4.1 window entry: 512 E4M3 values and 16 E8M0 scales, 528 B
    assert O.quant_rows(O.MXFP8, 512, 0, np.zeros((1, 512), np.float32)).shape == (1, 528)
    # X = 2^(floor(log2 amax) - 8): the block maximum lands in [256, 512) scale units
    assert O.mx8_scale(448.0) == 127 and O.mx8_scale(256.0) == 127 and O.mx8_scale(511.9) == 127
    assert O.mx8_scale(255.9) == 126 and O.mx8_scale(512.0) == 128 and O.mx8_scale(1.0) == 119
    assert O.mx8_scale(0.0) == 0 and O.mx8_scale(2.0 ** -140) == 0
    # one block encoded by hand: amax 1 -> X = 2^-8; 1 -> 256 = 2^8 (0 1111 000), -0.3 -> -76.8,
    # nearest 1.25 * 2^6 (1 1101 010), 0.5 -> 2^7 (0 1110 000), 2^-10 -> 2^-2 (0 0101 000)
    x = np.zeros((1, 32), np.float32)
    x[0, :4] = [1.0, -0.3, 0.5, 2.0 ** -10]
    r = O.quant_rows(O.MXFP8, 32, 0, x)
    assert list(r[0, :4]) == [0x78, 0xEA, 0x70, 0x28] and not r[0, 4:32].any() and r[0, 32] == 119
    # saturation: amax 511 -> X = 1, 511 clamps to 448 (0 1111 110)
    x[0, 0] = 511.0
    r = O.quant_rows(O.MXFP8, 32, 0, x)
    assert r[0, 32] == 127 and r[0, 0] == 0x7E


def test_mxfp8_row_roundtrip_and_error_bound():
    rng = np.random.default_rng(13)
    codes = rng.integers(0, 0x7F, (40, 128)).astype(np.uint32) | (rng.integers(0, 2, (40, 128)) << 7).astype(np.uint32)
    codes[:, ::32] = rng.integers(0x78, 0x7F, (40, 4))                   # 256 .. 448 in every block
    e = rng.integers(100, 150, (40, 4))
    x = (O.e4m3_value(codes) * np.repeat(2.0 ** (e - 127), 32, axis=1)).astype(np.float32)
    r = O.quant_rows(O.MXFP8, 128, 0, x)
    assert np.array_equal(O.dequant_rows(O.MXFP8, 128, 0, r), x)
    assert np.array_equal(r[:, 128:], e.astype(np.uint8))
    y = (rng.standard_normal((64, 128)) * rng.uniform(1e-3, 1e3, (64, 1))).astype(np.float32)
    ry = O.quant_rows(O.MXFP8, 128, 0, y)
    d = O.dequant_rows(O.MXFP8, 128, 0, ry)
    Xs = np.repeat(O.e8m0_value(ry[:, 128:]), 32, axis=1)
    small = np.abs(y) <= 448 * Xs                                        # E4M3 RNE: half an ulp
    assert np.all(np.abs(d - y)[small] <= np.maximum(2.0 ** -4 * np.abs(y), 2.0 ** -10 * Xs)[small])
    assert (~small).any() and np.all(np.abs(d[~small]) == 448 * Xs[~small])   # saturation
    assert not O.quant_rows(O.MXFP8, 128, 0, np.zeros((1, 128), np.float32)).any()
