"""Seeded input rows that put the quantisers on their rounding decisions.

Test infrastructure (inputs only, no arithmetic of the method): rows of fp32
values built so that, under each row format's scale rule, the value divided by
its block scale lands exactly on a midpoint between two neighbouring codes (or
one fp32 step beside one), so that the tie rule decides the code; and block
maxima whose scale itself is rounded from a midpoint.

Two families:
  grid rows  every value is k / 64 (k an integer), and the squares sum to exactly
             the row width in fp32 whatever the order of summation; an RMS
             normalisation with unit weight and eps 0 then leaves the row as it is,
             so the CSA2 compressor's entry equals the designed row bit for bit;
  ulp rows   no such constraint: block scales over many binades (subnormal E4M3
             scales and zero scales included), midpoints and their fp32 neighbours.
"""
import numpy as np

Q = 64.0                                   # grid rows: values k / Q

# E4M3 magnitudes (OCP fn): subnormals m * 2^-9, normals (1 + m/8) 2^(e-7)
E4M3_POS = np.array(sorted({m * 2.0 ** -9 for m in range(1, 8)} |
                           {(1 + m / 8) * 2.0 ** (e - 7) for e in range(1, 16) for m in range(8)
                            if not (e == 15 and m == 7)}))
E2M1_POS = np.array([0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _mids(grid):
    g = np.concatenate([[0.0], grid])
    return (g[:-1] + g[1:]) / 2


E4M3_MID = _mids(E4M3_POS)                 # 126 midpoints from 2^-10 up to 432
E2M1_MID = _mids(E2M1_POS)                 # 0.25 0.75 1.25 1.75 2.5 3.5 5


def _ulp_variants(v):
    v = np.asarray(v, np.float32)
    return np.concatenate([v, np.nextafter(v, np.float32(np.inf)), np.nextafter(v, np.float32(0))])


# ---- grid blocks: (block maximum k, element ks that land on midpoints) ----------
def _ks(values, scale):
    """k with k / Q = value * scale exactly (values on the Q-grid only)."""
    out = []
    for v in values:
        k = v * scale * Q
        if abs(k - round(k)) < 1e-12:
            out.append(int(round(k)))
    return out


def e4m3_grid_block():
    """An E4M3 128-block with maximum 7 (scale 7/448 = 2^-6: x / s = 64 x = k):
    E4M3 midpoints at integers (16 .. 432)."""
    kmax = 448
    mids = [int(m) for m in E4M3_MID if m >= 16 and m == int(m) and m < 448]
    return kmax, mids


def e2m1_grid_blocks():
    """E2M1 16-blocks: (block max k, midpoint element ks). The scale is
    E4M3(amax / 6); maxima 6, 3, 1.5 give scales 1, 1/2, 1/4; maxima 6 m for an
    E4M3 midpoint m round the scale itself (1.0625 -> 1, 1.1875 -> 1.25,
    0.53125 -> 0.5, 0.59375 -> 0.625, 0.65625 -> 0.625, 0.71875 -> 0.75)."""
    out = []
    for amax, s in ((6.0, 1.0), (3.0, 0.5), (1.5, 0.25), (6.375, 1.0), (7.125, 1.25), (3.1875, 0.5),
                    (3.5625, 0.625), (3.9375, 0.625), (4.3125, 0.75)):
        kmax = int(round(amax * Q))
        assert kmax == amax * Q
        ks = [k for k in _ks(E2M1_MID, s) if k < kmax]
        out.append((kmax, ks))
    return out


def mxfp4_grid_blocks():
    """MXFP4 32-blocks: maxima in [4, 8) take X = 1, in [2, 4) X = 1/2, [1, 2) X = 1/4."""
    out = []
    for amax, X in ((6.0, 1.0), (7.9375, 1.0), (4.0, 1.0), (3.0, 0.5), (1.5, 0.25)):
        kmax = int(amax * Q)
        out.append((kmax, [k for k in _ks(E2M1_MID, X) if k < kmax]))
    return out


def _fill_squares(rng, free, target):
    """Non-negative ks (at most 64) for the `free` channels whose squares sum to
    exactly `target`: random values around the mean still needed, then the last
    channels by greedy squares."""
    ks = np.zeros(free, np.int64)
    rem = target
    tail = min(24, free)
    if target > (free - 8) * 64 * 64:
        raise ValueError("target too large for the free channels")
    for i in range(free - tail):
        left = free - i                              # channels still free, this one included
        r = np.sqrt(rem / left)
        # at least what keeps the rest reachable (16 tail channels at 64^2, the last 8 for the exact remainder)
        need = rem - ((left - 1 - tail) + 16) * 64 * 64
        lo = max(int(0.8 * r), int(np.ceil(np.sqrt(need))) if need > 0 else 0)
        hi = min(64, int(1.2 * r) + 1, int(np.sqrt(rem)))
        k = int(rng.integers(min(lo, hi), hi + 1))
        ks[i] = k
        rem -= k * k
    for i in range(free - tail, free):
        k = min(64, int(np.sqrt(rem)))
        ks[i] = k
        rem -= k * k
    if rem != 0:
        raise ValueError("could not reach the target")
    return ks


def grid_row(rng, fmt, dim, rope, fmts):
    """One grid row for a main-row format (fmts: the format codes). Returns fp32 [dim + rope].
    A design whose free channels cannot reach the exact sum is drawn again."""
    for _ in range(1000):
        try:
            return _grid_row(rng, fmt, dim, rope, fmts)
        except ValueError as e:
            if "target" not in str(e):
                raise
    raise RuntimeError("no feasible grid row")


def _grid_row(rng, fmt, dim, rope, fmts):
    D = dim + rope
    target = int(Q * Q) * D                    # sum of k^2 for a mean square of 1
    k = np.zeros(D, np.int64)
    fixed = np.zeros(D, bool)
    if fmt == fmts["E4M3_S128"]:
        kmax, mids = e4m3_grid_block()
        rng.shuffle(mids)
        budget = 0.8 * target - (dim // 128) * kmax * kmax
        keep, used = [], 0
        for m in mids:                               # as many midpoints as the budget allows
            if used + m * m <= budget:
                keep.append(m)
                used += m * m
        mids = keep
        per = int(np.ceil(len(mids) / (dim // 128)))
        for blk in range(dim // 128):
            c0 = blk * 128
            k[c0] = kmax
            fixed[c0] = True
            m = mids[blk * per:(blk + 1) * per]
            k[c0 + 1:c0 + 1 + len(m)] = m
            fixed[c0 + 1:c0 + 1 + len(m)] = True
    else:
        if fmt == fmts["E2M1_S16"]:
            blocks, bs = e2m1_grid_blocks(), 16
        elif fmt == fmts["MXFP4"]:
            blocks, bs = mxfp4_grid_blocks(), 32
        else:
            raise ValueError("grid rows: E4M3_S128, E2M1_S16 or MXFP4")
        nb = dim // bs
        rem, free_ch = target, D
        for blk in range(nb):
            later = nb - blk - 1                     # later blocks, at least a maximum of 64 each
            kmax, ks = blocks[int(rng.integers(len(blocks)))]
            for cand in (list(ks)[:bs - 1], []):     # with its midpoints, else its maximum alone
                cost = kmax * kmax + sum(x * x for x in cand)
                r2, f2 = rem - cost - later * 4096, free_ch - 1 - len(cand) - later
                if 0 <= r2 <= (f2 - 8) * 4096:
                    break
            else:
                kmax, cand, cost = 64, [], 4096      # a plain block
            rem -= cost
            free_ch -= 1 + len(cand)
            c0 = blk * bs
            k[c0] = kmax
            k[c0 + 1:c0 + 1 + len(cand)] = cand
            fixed[c0:c0 + 1 + len(cand)] = True
    free = np.flatnonzero(~fixed)
    rem = target - int(np.sum(k * k))
    fill = _fill_squares(rng, len(free), rem)
    # fillers must stay at or below their block's maximum: they are at most 64, and every
    # block maximum is at least 64 (the E4M3 blocks' is 448; the RoPE tail has none)
    k[free] = fill
    sign = rng.choice([-1, 1], D)
    x = (sign * k).astype(np.float64) / Q
    assert np.sum(k * k) == target
    return x.astype(np.float32)


def ulp_row(rng, fmt, dim, rope, fmts):
    """One row of midpoints and their fp32 neighbours over many block scales."""
    D = dim + rope
    x = np.zeros(D, np.float64)
    if fmt == fmts["E4M3_S128"]:
        for c0 in range(0, dim, 128):
            e = int(rng.integers(-12, 13))
            sc = 2.0 ** e                            # amax = 448 * 2^e: scale 2^e exactly
            vals = rng.choice(_ulp_variants(np.concatenate([E4M3_MID, E4M3_POS])).astype(np.float64), 127)
            x[c0] = 448.0 * sc
            x[c0 + 1:c0 + 128] = vals * sc
    elif fmt == fmts["E2M1_S16"]:
        for c0 in range(0, dim, 16):
            kind = int(rng.integers(4))
            if kind == 0:                            # scale 2^e: amax 6 * 2^e
                sc = 2.0 ** int(rng.integers(-8, 7))
                amax = 6.0 * sc
            elif kind == 1:                          # amax / 6 on an E4M3 midpoint (subnormal ones included)
                m = float(rng.choice(E4M3_MID[E4M3_MID < 400]))
                amax = 6.0 * m
                sc = m
            elif kind == 2:                          # amax / 6 below half the smallest subnormal: zero scale
                amax = 6.0 * 2.0 ** -11
                sc = 2.0 ** -12
            else:                                    # scale saturates at 448; elements saturate at 6
                amax = 6.0 * 448.0 * 1.5
                sc = 448.0
            vals = rng.choice(_ulp_variants(np.concatenate([E2M1_MID, E2M1_POS])).astype(np.float64), 15)
            x[c0] = amax
            x[c0 + 1:c0 + 16] = np.minimum(vals * sc, amax)
    elif fmt == fmts["MXFP4"]:
        for c0 in range(0, dim, 32):
            e = int(rng.integers(-20, 20))
            X = 2.0 ** e
            x[c0] = float(rng.choice([4.0, 6.0, 7.99])) * X
            vals = rng.choice(_ulp_variants(np.concatenate([E2M1_MID, E2M1_POS])).astype(np.float64), 31)
            x[c0 + 1:c0 + 32] = vals * X
    elif fmt == fmts["MXFP8"]:
        for c0 in range(0, dim, 32):
            e = int(rng.integers(-30, 30))
            X = 2.0 ** e
            x[c0] = float(rng.choice([256.0, 448.0, 500.0])) * X
            vals = rng.choice(_ulp_variants(np.concatenate([E4M3_MID, E4M3_POS])).astype(np.float64), 31)
            x[c0 + 1:c0 + 32] = vals * X
    elif fmt == fmts["BF16"]:
        e = rng.integers(-20, 20, dim)
        m = rng.integers(0, 128, dim)
        x[:dim] = (1.0 + (2 * m + 1) / 256.0) * np.exp2(e)        # bf16 midpoints
    else:
        raise ValueError(fmt)
    if rope:                                          # bf16 RoPE tail: bf16 midpoints and neighbours
        e = rng.integers(-10, 10, rope)
        m = rng.integers(0, 128, rope)
        x[dim:] = (1.0 + (2 * m + 1) / 256.0) * np.exp2(e)
    x *= rng.choice([-1.0, 1.0], D)
    x = x.astype(np.float32)
    nudge = rng.integers(-1, 2, D)                   # fp32 neighbours of a third of the RoPE midpoints
    if rope:
        t = x[dim:]
        t[nudge[dim:] > 0] = np.nextafter(t[nudge[dim:] > 0], np.float32(np.inf))
        t[nudge[dim:] < 0] = np.nextafter(t[nudge[dim:] < 0], np.float32(0))
    return x
