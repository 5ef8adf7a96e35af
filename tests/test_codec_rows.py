"""The midpoint rows the GPU codec tests feed (tests/codec_rows.py) really put
the quantisers on their rounding decisions: under each format's scale rule (the
oracle's), many values divided by their block scale sit exactly halfway
between two codes; block maxima round their own E4M3 scale from a midpoint; and
grid rows keep a mean square of exactly 1 in fp32 in any summation order. CPU only."""
import numpy as np

import oracle as O
from tests import codec_rows as R

FM = {"E4M3_S128": O.E4M3_S128, "E2M1_S16": O.E2M1_S16, "MXFP4": O.MXFP4, "MXFP8": O.MXFP8, "BF16": O.BF16}


def _blocks(x, bs):
    return x.reshape(-1, bs)


def _count_e4m3_mid(q):
    return int(np.isin(np.abs(q).astype(np.float64), R.E4M3_MID).sum())


def _count_e2m1_mid(q):
    return int(np.isin(np.abs(q).astype(np.float64), R.E2M1_MID).sum())


def test_grid_rows_have_unit_mean_square_in_any_order():
    rng = np.random.default_rng(1)
    for fmt, dim, rope in ((O.E4M3_S128, 512, 64), (O.E2M1_S16, 512, 0), (O.MXFP4, 128, 0)):
        for _ in range(20):
            x = R.grid_row(rng, fmt, dim, rope, FM)
            for order in (np.arange(x.size), rng.permutation(x.size)):
                s = np.float32(0)
                for v in x[order]:
                    s = np.float32(s + np.float32(v) * np.float32(v))
                assert s == np.float32(dim + rope)


def test_e4m3_rows_hit_midpoints():
    rng = np.random.default_rng(2)
    hits = 0
    for fam in (R.grid_row, R.ulp_row):
        for _ in range(20):
            x = fam(rng, O.E4M3_S128, 512, 64, FM)[:512]
            for b in _blocks(x, 128):
                s = np.float32(np.abs(b).max()) / np.float32(448.0)     # the V3.2 scale rule
                hits += _count_e4m3_mid(b / s)
    assert hits > 1000


def test_e2m1_rows_hit_midpoints_and_scale_midpoints():
    rng = np.random.default_rng(3)
    hits = scale_ties = zero_scales = 0
    for fam in (R.grid_row, R.ulp_row):
        for _ in range(40):
            x = fam(rng, O.E2M1_S16, 512, 0, FM)
            for b in _blocks(x, 16):
                a6 = np.float32(np.abs(b).max()) / np.float32(6.0)
                scale_ties += _count_e4m3_mid(np.array([a6]))
                s = O.e4m3_value(O.e4m3_encode(np.array([a6], np.float32)))[0]
                if s == 0:
                    zero_scales += 1
                    continue
                hits += _count_e2m1_mid(b / np.float32(s))
    assert hits > 1000 and scale_ties > 50 and zero_scales > 5


def test_mx_rows_hit_midpoints():
    rng = np.random.default_rng(4)
    h4 = h8 = 0
    for _ in range(40):
        for fam in (R.grid_row, R.ulp_row):
            x = fam(rng, O.MXFP4, 128, 0, FM)
            for b in _blocks(x, 32):
                X = O.e8m0_value(np.array([O.mx_scale(np.abs(b).max())], np.uint8))[0]
                h4 += _count_e2m1_mid(b / np.float32(X))
        x = R.ulp_row(rng, O.MXFP8, 512, 0, FM)
        for b in _blocks(x, 32):
            X = O.e8m0_value(np.array([O.mx8_scale(np.abs(b).max())], np.uint8))[0]
            h8 += _count_e4m3_mid(b / np.float32(X))
    assert h4 > 500 and h8 > 500


def test_bf16_rows_hit_midpoints():
    rng = np.random.default_rng(5)
    x = R.ulp_row(rng, O.BF16, 512, 64, FM).astype(np.float32)
    low = x.view(np.uint32) & 0xFFFF
    assert np.sum(low == 0x8000) > 300                    # exactly halfway between two bf16 values
