"""The CSA2 compressor at append on the GPU against the oracle: the fp32 entry
(gated softmax pooling over the window's m tokens, RMS normalisation, forward
RoPE) within fp32 rounding, rows written only at their slots, the quantised
row equal byte for byte to the oracle's quantisation of the GPU's own fp32
entry, and to the oracle's whole path where the entry is exactly representable."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_latent_attention_mla_amd as M

pytestmark = pytest.mark.gpu
DEV = "cuda"

# (name, row format, dim, rope, B, m, rotated channels)
CASES = [
    ("v41_m2_e2m1", M.E2M1_S16, 512, 0, 4, 2, 64),
    ("v4_m4_e4m3_rope", M.E4M3_S128, 512, 64, 2, 4, 64),
    ("m128_bf16", M.BF16, 512, 0, 1, 128, 0),
    ("m1_f32", M.F32, 64, 16, 3, 1, 16),
    ("m3_mxfp4", M.MXFP4, 128, 0, 2, 3, 0),
]
ORC_FMT = {M.F32: O.F32, M.BF16: O.BF16, M.E4M3_S128: O.E4M3_S128, M.E2M1_S16: O.E2M1_S16, M.MXFP4: O.MXFP4}


def _run(fmt, dim, rope, kv, gate, g, eps, cs, slots, cap):
    B, m, D = kv.shape
    row = M.Row(fmt, dim, rope)
    cache = torch.zeros((B, cap, M.row_bytes(row)), dtype=torch.uint8, device=DEV)
    out = torch.empty((B, D), dtype=torch.float32, device=DEV)
    t = lambda x: None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    M.mla_compress_append(row, t(kv), t(gate), cache, t(slots), t(g), eps, t(cs), out)
    torch.cuda.synchronize()
    return out.cpu().numpy(), cache.cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_compress_matches_the_oracle(case):
    name, fmt, dim, rope, B, m, r = case
    print("compress", name, flush=True)
    D = dim + rope
    rng = np.random.default_rng(len(name) * 7 + m)
    kv = rng.standard_normal((B, m, D)).astype(np.float32)
    gate = (rng.standard_normal((B, m, D)) * 2).astype(np.float32)
    g = rng.uniform(0.5, 1.5, D).astype(np.float32)
    th = rng.uniform(0, 6.3, (B, r // 2))
    cs = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32) if r else None
    cap = 5
    slots = np.array([(3 * b + 1) % cap for b in range(B)], np.int32)
    got, cache = _run(fmt, dim, rope, kv, gate, g, 1e-6, cs, slots, cap)
    ref = O.compress(kv, gate, g, 1e-6, rope_cs=cs)
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)
    want = O.quant_rows(ORC_FMT[fmt], dim, rope, ref)
    for b in range(B):
        assert not np.delete(cache[b], slots[b], axis=0).any(), "only the entry's row is written"
    rows = cache[np.arange(B), slots]
    # the quantised row is the oracle's quantisation of the GPU's own fp32 entry, byte for byte
    assert np.array_equal(rows, O.quant_rows(ORC_FMT[fmt], dim, rope, got)), "rows differ from quant(out_entry)"
    if fmt == M.F32:
        assert np.array_equal(rows.view(np.float32), got)


@pytest.mark.parametrize("fmt", [M.E2M1_S16, M.E4M3_S128])
def test_compress_masked_gates(fmt):
    """Gates of -inf (masked window slots, as an overlapping compressor initialises
    them) weigh zero: leading, interleaved and trailing -inf gates, with at least one
    finite gate per channel, give the oracle's finite entry."""
    dim, rope = (512, 64) if fmt == M.E4M3_S128 else (512, 0)
    D, B, m = dim + rope, 3, 4
    rng = np.random.default_rng(77 + fmt)
    kv = rng.standard_normal((B, m, D)).astype(np.float32)
    gate = rng.standard_normal((B, m, D)).astype(np.float32)
    gate[0, :3] = -np.inf                                # only the last token counts
    gate[1, 0] = -np.inf                                 # the first token masked
    gate[1, 2, ::3] = -np.inf
    gate[2, 1:] = -np.inf                                # only the first token counts
    g = rng.uniform(0.5, 1.5, D).astype(np.float32)
    slots = np.array([0, 1, 2], np.int32)
    got, cache = _run(fmt, dim, rope, kv, gate, g, 1e-6, None, slots, 3)
    ref = O.compress(kv, gate, g, 1e-6)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-5, atol=1e-5)
    assert np.array_equal(cache[np.arange(B), slots], O.quant_rows(ORC_FMT[fmt], dim, rope, got))


@pytest.mark.parametrize("fmt", [M.E2M1_S16, M.E4M3_S128, M.BF16, M.MXFP4])
def test_compress_bytes_exact_when_the_entry_is_representable(fmt):
    """Equal gates (weights 1/m exactly at m = 2), |kv| a power of two per
    sequence, power-of-two weights and eps = 0: every step is exact in fp32,
    so the quantised rows must equal the oracle's byte for byte."""
    dim, rope = (512, 64) if fmt == M.E4M3_S128 else (512, 0)
    D, B, m = dim + rope, 3, 2
    rng = np.random.default_rng(fmt)
    sgn = rng.choice([-1.0, 1.0], (B, 1, D))
    kv = np.repeat(sgn * np.exp2(rng.integers(-4, 4, (B, 1, 1))), m, axis=1).astype(np.float32)
    gate = np.repeat(rng.standard_normal((B, 1, D)), m, axis=1).astype(np.float32)
    g = np.exp2(rng.integers(-3, 4, D)).astype(np.float32)
    slots = np.array([0, 2, 1], np.int32)
    got, cache = _run(fmt, dim, rope, kv, gate, g, 0.0, None, slots, 3)
    ref = O.compress(kv, gate, g, 0.0)
    assert np.array_equal(got, ref)
    want = O.quant_rows(ORC_FMT[fmt], dim, rope, ref)
    assert np.array_equal(cache[np.arange(B), slots], want)
