"""Pins of the oracle's indexer, top-k and attention to things outside the
oracle: special cases that reduce to library routines, identities, the pages'
absorption worked example, invariants.  CPU only."""
import json
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle as O
import workloads as WL

E4M3_GRID = None


def _exact_e4m3_keys(rng, n, dim):
    """Keys made of E4M3 grid values with one +-448 per 128-block: the block
    scale is exactly 1, so the quantised row decodes to the input exactly."""
    global E4M3_GRID
    if E4M3_GRID is None:
        v = O.e4m3_value(np.arange(0x7F))
        E4M3_GRID = v[v <= 64]
    x = rng.choice(E4M3_GRID, (n, dim)) * rng.choice([-1, 1], (n, dim))
    x[:, ::128] = 448.0
    return x.astype(np.float32)


def _exact_fp4_keys(rng, n, dim):
    lad = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    x = rng.choice(lad, (n, dim)) * rng.choice([-1, 1], (n, dim))
    x[:, ::16] = 6.0                                             # scale E4M3(1.0) = 1
    return x.astype(np.float32)


def _exact_mx_keys(rng, n, dim):
    lad = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    x = rng.choice(lad, (n, dim)) * rng.choice([-1, 1], (n, dim))
    x[:, ::32] = 6.0                                             # E8M0 scale 2^0
    return x.astype(np.float32)


KEY_MAKERS = {
    O.F32: lambda rng, n, d: rng.standard_normal((n, d)).astype(np.float32),
    O.E4M3_S128: _exact_e4m3_keys,
    O.E2M1_S16: _exact_fp4_keys,
    O.MXFP4: _exact_mx_keys,
}


@pytest.mark.parametrize("fmt,dim", [(O.F32, 32), (O.E4M3_S128, 128), (O.E2M1_S16, 128)])
def test_indexer_single_head_reduces_to_relu_of_dot(fmt, dim):
    rng = np.random.default_rng(10)
    N, H_I = 300, 3
    keys = KEY_MAKERS[fmt](rng, N, dim)
    rows = O.quant_rows(fmt, dim, 0, keys)[None]
    assert np.array_equal(O.dequant_rows(fmt, dim, 0, rows)[0], keys)       # exact keys
    q = rng.standard_normal((1, H_I, dim)).astype(np.float32)
    sigma = dim ** -0.5
    for j in range(H_I):                                  # one-hot weight on head j
        w = np.zeros((1, H_I), np.float32)
        w[0, j] = 1.0
        got = O.indexer_scores((fmt, dim, 0), q, w, sigma, rows, [N])[0]
        ref = np.maximum(sigma * (keys.astype(np.float64) @ q[0, j].astype(np.float64)), 0)
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)


def test_mxfp4_indexer_quantises_the_query_too():
    """With MXFP4 keys the query-key product runs in FP4: a query on the MXFP4
    grid scores as ReLU(sigma q.k) exactly (np.dot), and any query scores as its
    own MXFP4 rounding (which differs from the unrounded query's score)."""
    rng = np.random.default_rng(13)
    N, H_I, dim = 200, 3, 128
    keys = _exact_fp4_keys(rng, N, dim)                  # on both grids (a 6 in every 16 channels)
    rows = O.quant_rows(O.MXFP4, dim, 0, keys)[None]
    assert np.array_equal(O.dequant_rows(O.MXFP4, dim, 0, rows)[0], keys)
    sigma = dim ** -0.5
    q_grid = (_exact_mx_keys(rng, H_I, dim) * np.float32(0.25))[None]       # scale 2^-2, still on the grid
    for j in range(H_I):
        w = np.zeros((1, H_I), np.float32)
        w[0, j] = 1.0
        got = O.indexer_scores((O.MXFP4, dim, 0), q_grid, w, sigma, rows, [N])[0]
        ref = np.maximum(sigma * (keys.astype(np.float64) @ q_grid[0, j].astype(np.float64)), 0)
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)
    q = rng.standard_normal((1, H_I, dim)).astype(np.float32)
    q_hat = O.dequant_rows(O.MXFP4, dim, 0, O.quant_rows(O.MXFP4, dim, 0, q[0]))[None].astype(np.float32)
    w = rng.standard_normal((1, H_I)).astype(np.float32)
    s_q = O.indexer_scores((O.MXFP4, dim, 0), q, w, sigma, rows, [N])
    assert np.array_equal(s_q, O.indexer_scores((O.MXFP4, dim, 0), q_hat, w, sigma, rows, [N]))
    # the unrounded query through the E2M1 format (which leaves queries alone) scores differently
    rows16 = O.quant_rows(O.E2M1_S16, dim, 0, keys)[None]
    assert np.array_equal(O.dequant_rows(O.E2M1_S16, dim, 0, rows16)[0], keys)
    assert not np.array_equal(s_q, O.indexer_scores((O.E2M1_S16, dim, 0), q, w, sigma, rows16, [N]))
    np.testing.assert_allclose(s_q, O.indexer_scores((O.E2M1_S16, dim, 0), q_hat, w, sigma, rows16, [N]),
                               rtol=1e-6, atol=1e-7)


def test_indexer_relu_difference_is_the_bilinear_form():
    # ReLU(x) - ReLU(-x) = x, so I(q) - I(-q) = sum_j w_j sigma q_j . k
    rng = np.random.default_rng(11)
    B, N, H_I, d = 2, 500, 8, 32
    keys = rng.standard_normal((B, N, d)).astype(np.float32)
    rows = O.quant_rows(O.F32, d, 0, keys)
    q = rng.standard_normal((B, H_I, d)).astype(np.float32)
    w = rng.standard_normal((B, H_I)).astype(np.float32)
    sigma = d ** -0.5
    a = O.indexer_scores((O.F32, d, 0), q, w, sigma, rows, [N, N]).astype(np.float64)
    b = O.indexer_scores((O.F32, d, 0), -q, w, sigma, rows, [N, N]).astype(np.float64)
    ref = sigma * np.einsum("bj,bjc,bnc->bn", w.astype(np.float64), q.astype(np.float64),
                            keys.astype(np.float64))
    np.testing.assert_allclose(a - b, ref, rtol=1e-5, atol=1e-5)
    # and I(q) + I(-q) = sum_j w_j sigma |q_j . k|
    ref_abs = sigma * np.einsum("bj,bjn->bn", w.astype(np.float64),
                                np.abs(np.einsum("bjc,bnc->bjn", q.astype(np.float64),
                                                 keys.astype(np.float64))))
    np.testing.assert_allclose(a + b, ref_abs, rtol=1e-5, atol=1e-5)


def test_indexer_votes_nonnegative_and_linear_in_weights():
    rng = np.random.default_rng(12)
    N, H_I, d = 400, 6, 32
    keys = rng.standard_normal((1, N, d)).astype(np.float32)
    rows = O.quant_rows(O.F32, d, 0, keys)
    q = rng.standard_normal((1, H_I, d)).astype(np.float32)
    w1 = np.abs(rng.standard_normal((1, H_I))).astype(np.float32)
    s1 = O.indexer_scores((O.F32, d, 0), q, w1, 0.17, rows, [N])
    assert np.all(s1 >= 0)                                 # non-negative votes
    w2 = rng.standard_normal((1, H_I)).astype(np.float32)
    s2 = O.indexer_scores((O.F32, d, 0), q, w2, 0.17, rows, [N])
    s12 = O.indexer_scores((O.F32, d, 0), q, w1 + w2, 0.17, rows, [N])
    np.testing.assert_allclose(s12, s1.astype(np.float64) + s2, rtol=1e-5, atol=1e-6)


def test_indexer_causal_mask_and_candidate_pool():
    rng = np.random.default_rng(13)
    B, N, H_I, d = 2, 200, 4, 128
    keys = rng.standard_normal((B, N, d)).astype(np.float32)
    rows = O.quant_rows(O.E4M3_S128, d, 0, keys)
    q = rng.standard_normal((B, H_I, d)).astype(np.float32)
    w = rng.standard_normal((B, H_I)).astype(np.float32)
    full = O.indexer_scores((O.E4M3_S128, d, 0), q, w, d ** -0.5, rows, [N, N])
    part = O.indexer_scores((O.E4M3_S128, d, 0), q, w, d ** -0.5, rows, [77, 0])
    assert np.array_equal(part[0, :77], full[0, :77])
    assert np.all(np.isneginf(part[0, 77:])) and np.all(np.isneginf(part[1]))
    cand = np.stack([rng.permutation(N)[:50], rng.permutation(N)[:50]]).astype(np.int32)
    cand[0, :3] = [-1, 150, 199]
    pool = O.indexer_scores((O.E4M3_S128, d, 0), q, w, d ** -0.5, rows, [120, N], cand=cand)
    for b, nv in ((0, 120), (1, N)):
        for i, s in enumerate(cand[b]):
            if 0 <= s < nv:
                assert pool[b, i] == full[b, s]
            else:
                assert np.isneginf(pool[b, i])


def _lexsort_topk(scores, nvis, k):
    pos = np.arange(nvis)
    order = np.lexsort((pos, -scores[:nvis].astype(np.float64)))   # score desc, position asc
    sel = list(pos[order[:k]])
    return sel + [-1] * (k - len(sel))


def test_topk_matches_library_sort_with_ties_and_padding():
    rng = np.random.default_rng(14)
    B, N = 3, 1000
    scores = rng.integers(-20, 20, (B, N)).astype(np.float32) * 0.25     # many exact ties
    nvis = np.array([1000, 333, 5], np.int32)
    for k in (1, 7, 100, 333, 400):
        got = O.topk(scores, nvis, k)
        for b in range(B):
            assert list(got[b]) == _lexsort_topk(scores[b], nvis[b], k)


def test_topk_k_at_least_visible_selects_all_visible():
    rng = np.random.default_rng(15)
    scores = rng.standard_normal((2, 64)).astype(np.float32)
    got = O.topk(scores, np.array([64, 20], np.int32), 80)
    assert sorted(got[0][got[0] >= 0]) == list(range(64)) and np.sum(got[0] < 0) == 16
    assert sorted(got[1][got[1] >= 0]) == list(range(20)) and np.sum(got[1] < 0) == 60


def test_topk_with_candidate_pool_returns_positions():
    rng = np.random.default_rng(16)
    scores = rng.standard_normal((1, 10)).astype(np.float32)
    cand = np.array([[90, 3, -1, 40, 7, 500, 12, 13, 14, 15]], np.int32)
    got = O.topk(scores, np.array([100], np.int32), 4, n_rows=100, cand=cand)
    legal = [i for i in range(10) if 0 <= cand[0, i] < 100]
    best = sorted(legal, key=lambda i: (-scores[0, i], cand[0, i]))[:4]
    assert list(got[0]) == [int(cand[0, i]) for i in best]


# ---- candidate pool (hierarchical sparse indexer) -------------------------
def test_pool_hand_fixture():
    """Blocks of 4 over 14 positions, 11 visible: block 0 scores 9, block 1
    scores 7, block 2 scores 8 (positions 8 .. 10; the 12s lie past n_visible),
    block 3 has no visible position; so the pool is 0, 2, 1, then -1."""
    s = np.array([[1, 9, 2, 3, 0, 5, 7, 6, 8, -1, 4, 12, 12, 3]], np.float32)
    nv = np.array([11], np.int32)
    assert O.pool(s, nv, 3, block=4).tolist() == [[0, 2, 1]]
    assert O.pool(s, nv, 5, block=4).tolist() == [[0, 2, 1, -1, -1]]
    assert O.pool(s, nv, 2, block=4).tolist() == [[0, 2]]
    # equal maxima: the smaller block first
    t = np.array([[5, 1, 2, 5, 0, 0]], np.float32)
    assert O.pool(t, np.array([6], np.int32), 3, block=2).tolist() == [[0, 1, 2]]
    assert O.pool(t, np.array([6], np.int32), 1, block=3).tolist() == [[0]]


def test_pool_of_block_one_is_the_topk():
    rng = np.random.default_rng(21)
    s = rng.standard_normal((3, 300)).astype(np.float32)
    s[1, 10:20] = 0.5                                   # ties
    nv = np.array([300, 123, 7], np.int32)
    for n in (1, 40, 300):
        assert np.array_equal(O.pool(s, nv, n, block=1), O.topk(s, nv, n))


def test_pool_keeps_every_visible_block_and_contains_the_topk():
    rng = np.random.default_rng(22)
    B, N, blk = 4, 1000, 8
    s = rng.standard_normal((B, N)).astype(np.float32)
    nv = np.array([1000, 997, 9, 0], np.int32)
    everything = O.pool(s, nv, N // blk + 5, block=blk)
    for b in range(B):
        vis_blocks = (int(nv[b]) + blk - 1) // blk
        got = everything[b]
        assert sorted(got[got >= 0].tolist()) == list(range(vis_blocks))
        assert np.all(got[vis_blocks:] == -1)
    for n_blocks, k in ((20, 20), (20, 7), (64, 64)):
        pool = O.pool(s, nv, n_blocks, block=blk)
        top = O.topk(s, nv, k)
        for b in range(B):
            members = {int(p) for p in O.pool_positions(pool[b:b + 1], blk)[0] if p >= 0}
            assert {int(p) for p in top[b] if p >= 0} <= members


# ---- attention -------------------------------------------------------------
def test_absorbed_attention_equals_naive_mla_pages_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "absorption_worked_example.json")))
    rng = np.random.default_rng(0)
    d, n_h, d_h, d_c, T = 64, 4, 16, 32, 10
    W_DKV = rng.standard_normal((d_c, d)) / np.sqrt(d)
    W_UK = rng.standard_normal((n_h, d_h, d_c)) / np.sqrt(d_c)
    W_UV = rng.standard_normal((n_h, d_h, d_c)) / np.sqrt(d_c)
    W_Q = rng.standard_normal((n_h, d_h, d)) / np.sqrt(d)
    Hs = rng.standard_normal((T, d))
    h_t = rng.standard_normal(d)
    C = (Hs @ W_DKV.T).astype(np.float32).astype(np.float64)     # cached latents (fp32 rows)
    # naive MLA: per-head keys and values up-projected for every cached token
    K = np.einsum("hdc,tc->htd", W_UK, C)
    V = np.einsum("hdc,tc->htd", W_UV, C)
    q = np.einsum("hdk,k->hd", W_Q, h_t)
    p = softmax(np.einsum("hd,htd->ht", q, K), axis=1)
    out_naive = np.einsum("ht,htd->hd", p, V)
    # absorbed, through the oracle: q_abs = W_UK^T q over raw latents, W_UV after
    q_abs = np.einsum("hdc,hd->hc", W_UK, q).astype(np.float32)
    rows = O.quant_rows(O.F32, d_c, 0, C.astype(np.float32))[None]
    o_lat, lse = O.attention((O.F32, d_c, 0), d_c, q_abs[None], rows, np.arange(T, dtype=np.int32)[None], 1.0)
    out_abs = np.einsum("hdc,hc->hd", W_UV, o_lat[0].astype(np.float64))
    # fp32 q_abs and fp32 outputs: agreement at fp32 rounding level (page: fp64 level)
    scale = np.abs(out_naive).max()
    assert np.abs(out_abs - out_naive).max() <= 1e-5 * scale
    assert g["printed"]["max_abs_output_diff"] < 1e-12
    ref_lse = logsumexp(np.einsum("hc,tc->ht", q_abs.astype(np.float64), C), axis=1)
    np.testing.assert_allclose(lse[0], ref_lse, rtol=1e-6)


def test_absorbed_with_decoupled_rope_equals_naive_mla():
    # key = [W_UK c ; k_R] per head, value = W_UV c; absorbed rows are [c ; k_R]
    rng = np.random.default_rng(21)
    B, n_h, d_h, d_c, d_r, N, k = 2, 8, 16, 64, 16, 300, 64
    C = rng.standard_normal((B, N, d_c)).astype(np.float32).astype(np.float64)
    KR = rng.standard_normal((B, N, d_r)).astype(np.float32).astype(np.float64)
    W_UK = rng.standard_normal((n_h, d_h, d_c)) / np.sqrt(d_c)
    W_UV = rng.standard_normal((n_h, d_h, d_c)) / np.sqrt(d_c)
    q_nope = rng.standard_normal((B, n_h, d_h))
    q_rope = rng.standard_normal((B, n_h, d_r)).astype(np.float32).astype(np.float64)
    idx = np.stack([rng.permutation(N)[:k] for _ in range(B)]).astype(np.int32)
    sc = (d_h + d_r) ** -0.5
    q_abs = np.concatenate([np.einsum("hdc,bhd->bhc", W_UK, q_nope), q_rope], -1).astype(np.float32)
    rows = O.quant_rows(O.F32, d_c, d_r, np.concatenate([C, KR], -1).astype(np.float32))
    o_lat, lse = O.attention((O.F32, d_c, d_r), d_c, q_abs, rows, idx, sc)
    for b in range(B):
        sel = idx[b]
        Kn = np.einsum("hdc,tc->htd", W_UK, C[b, sel])
        Vn = np.einsum("hdc,tc->htd", W_UV, C[b, sel])
        s = (np.einsum("hd,htd->ht", q_nope[b], Kn) + q_rope[b] @ KR[b, sel].T) * sc
        # the oracle saw q_abs rounded to fp32: compare against that rounding's effect
        out_naive = np.einsum("ht,htd->hd", softmax(s, axis=1), Vn)
        out_abs = np.einsum("hdc,hc->hd", W_UV, o_lat[b].astype(np.float64))
        assert np.abs(out_abs - out_naive).max() <= 2e-5 * np.abs(out_naive).max()
        np.testing.assert_allclose(lse[b], logsumexp(s, axis=1), rtol=2e-6, atol=2e-6)


def _dense_reference(Kv, q, d_v, scale):
    s = scale * (q.astype(np.float64) @ Kv.T)
    return softmax(s, axis=-1) @ Kv[:, :d_v], logsumexp(s, axis=-1)


@pytest.mark.parametrize("fmt,dim,rope,d_v", [(O.E4M3_S128, 512, 64, 512), (O.E2M1_S16, 512, 0, 512),
                                              (O.BF16, 128, 32, 128), (O.F32, 64, 16, 64)])
def test_sparse_equals_dense_when_topk_covers_everything(fmt, dim, rope, d_v):
    rng = np.random.default_rng(22)
    B, H, N = 2, 4, 96
    x = rng.standard_normal((B, N, dim + rope)).astype(np.float32)
    rows = O.quant_rows(fmt, dim, rope, x)
    q = WL.bf16_round(rng.standard_normal((B, H, dim + rope)).astype(np.float32))
    keys = rng.standard_normal((B, N, 32)).astype(np.float32)
    irows = O.quant_rows(O.F32, 32, 0, keys)
    s = O.indexer_scores((O.F32, 32, 0), rng.standard_normal((B, 2, 32)), np.ones((B, 2)), 1.0, irows, [N, N])
    idx = O.topk(s, np.array([N, N], np.int32), N + 10)               # k >= T: everything
    out, lse = O.attention((fmt, dim, rope), d_v, q, rows, idx, 0.05)
    for b in range(B):
        Kv = O.dequant_rows(fmt, dim, rope, rows[b])
        ro, rl = _dense_reference(Kv, q[b], d_v, 0.05)
        np.testing.assert_allclose(out[b], ro, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(lse[b], rl, rtol=1e-6)


def test_lse_merge_of_a_partition_equals_the_whole_and_order_is_irrelevant():
    rng = np.random.default_rng(23)
    B, H, N, k = 1, 6, 200, 80
    x = rng.standard_normal((B, N, 288 * 0 + 512)).astype(np.float32)
    rows = O.quant_rows(O.E2M1_S16, 512, 0, x)
    q = rng.standard_normal((B, H, 512)).astype(np.float32)
    idx = rng.permutation(N)[:k].astype(np.int32)[None]
    o, l = O.attention((O.E2M1_S16, 512, 0), 512, q, rows, idx, 0.07)
    o1, l1 = O.attention((O.E2M1_S16, 512, 0), 512, q, rows, idx[:, :30], 0.07)
    o2, l2 = O.attention((O.E2M1_S16, 512, 0), 512, q, rows, idx[:, 30:], 0.07)
    lm = np.logaddexp(l1.astype(np.float64), l2)
    om = (np.exp(l1 - lm)[..., None] * o1 + np.exp(l2 - lm)[..., None] * o2)
    np.testing.assert_allclose(l, lm, rtol=1e-6)
    np.testing.assert_allclose(o, om, rtol=1e-5, atol=1e-6)
    op, lp = O.attention((O.E2M1_S16, 512, 0), 512, q, rows, idx[:, ::-1].copy(), 0.07)
    np.testing.assert_allclose(op, o, rtol=1e-6, atol=1e-7)
    assert np.allclose(lp, l, rtol=1e-7)
    # -1 entries are skipped; a repeated index counts twice (multiset)
    pad = np.concatenate([idx, -np.ones((1, 5), np.int32)], 1)
    o3, l3 = O.attention((O.E2M1_S16, 512, 0), 512, q, rows, pad, 0.07)
    np.testing.assert_allclose(o3, o, rtol=1e-6, atol=1e-7)
    dup = np.concatenate([idx, idx[:, :1]], 1)
    o4, l4 = O.attention((O.E2M1_S16, 512, 0), 512, q, rows, dup, 0.07)
    Kv = O.dequant_rows(O.E2M1_S16, 512, 0, rows[0])[dup[0]]
    ro, rl = _dense_reference(Kv, q[0], 512, 0.07)
    np.testing.assert_allclose(o4[0], ro, rtol=1e-5, atol=1e-6)


def test_window_branch_and_empty_set():
    rng = np.random.default_rng(24)
    B, H, N, W = 2, 4, 50, 16
    x = rng.standard_normal((B, N, 512)).astype(np.float32)
    rows = O.quant_rows(O.E2M1_S16, 512, 0, x)
    q = rng.standard_normal((B, H, 512)).astype(np.float32)
    wf = rng.standard_normal((B, W, 512)).astype(np.float32)
    ring = O.bf16_encode(wf)
    wl = np.array([16, 5], np.int32)
    none = -np.ones((B, 4), np.int32)
    o, l = O.attention((O.E2M1_S16, 512, 0), 512, q, rows, none, 0.05, ring, wl)
    for b in range(B):
        Kv = O.bf16_value(ring[b, :wl[b]]).astype(np.float64)
        ro, rl = _dense_reference(Kv, q[b], 512, 0.05)
        np.testing.assert_allclose(o[b], ro, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(l[b], rl, rtol=1e-6)
    # selected rows plus window = one softmax over the concatenation
    idx = np.stack([rng.permutation(N)[:10] for _ in range(B)]).astype(np.int32)
    o2, l2 = O.attention((O.E2M1_S16, 512, 0), 512, q, rows, idx, 0.05, ring, wl)
    for b in range(B):
        Kv = np.concatenate([O.dequant_rows(O.E2M1_S16, 512, 0, rows[b][idx[b]]),
                             O.bf16_value(ring[b, :wl[b]]).astype(np.float64)])
        ro, rl = _dense_reference(Kv, q[b], 512, 0.05)
        np.testing.assert_allclose(o2[b], ro, rtol=1e-5, atol=1e-6)
    # empty set: lse -inf, o = 0
    o3, l3 = O.attention((O.E2M1_S16, 512, 0), 512, q, rows, none, 0.05, ring, np.zeros(B, np.int32))
    assert np.all(np.isneginf(l3)) and np.all(o3 == 0)


def test_attention_sinks_follow_the_pages_formulation():
    """Attention sinks: one logit per head appended to the scaled scores as an
    extra column before the softmax and dropped after it (the pages' concat /
    softmax / slice), brute force with the library softmax; a -inf sink is the
    plain softmax; the relation to the sink-free result; an empty set keeps all
    mass on the sink (lse = sink, out = 0)."""
    rng = np.random.default_rng(29)
    B, H, N, k, scale = 1, 5, 60, 25, 0.09
    x = rng.standard_normal((B, N, 64)).astype(np.float32)
    rows = O.quant_rows(O.F32, 64, 0, x)                         # exact rows
    q = rng.standard_normal((B, H, 64)).astype(np.float32)
    idx = rng.permutation(N)[:k].astype(np.int32)[None]
    sinks = np.array([-1.5, 0.0, 2.0, 30.0, -np.inf], np.float32)
    o, l = O.attention((O.F32, 64, 0), 64, q, rows, idx, scale, sinks=sinks)
    K = x[0, idx[0]].astype(np.float64)
    for h in range(H):
        z = scale * (K @ q[0, h].astype(np.float64))
        p = softmax(np.concatenate([z, [float(sinks[h])]]))[:-1]
        np.testing.assert_allclose(o[0, h], p @ K, rtol=1e-5, atol=1e-7)
        np.testing.assert_allclose(l[0, h], logsumexp(np.concatenate([z, [float(sinks[h])]])), rtol=1e-6)
    o0, l0 = O.attention((O.F32, 64, 0), 64, q, rows, idx, scale)
    assert np.array_equal(o[0, 4], o0[0, 4]) and l[0, 4] == l0[0, 4]          # -inf sink = none
    ls = np.logaddexp(l0.astype(np.float64), sinks.astype(np.float64)[None])
    np.testing.assert_allclose(l, ls, rtol=1e-6)
    np.testing.assert_allclose(o, o0 * np.exp(l0 - ls)[..., None], rtol=1e-5, atol=1e-7)
    assert np.abs(o[0, 3]).max() < 1e-6 * np.abs(o0[0, 3]).max()               # a dominant sink
    oe, le = O.attention((O.F32, 64, 0), 64, q, rows, -np.ones((1, 4), np.int32), scale, sinks=sinks)
    assert np.all(oe == 0) and np.array_equal(le[0], sinks)


def test_output_rope_undoes_the_rotation_at_the_query_position():
    """O-RoPE: the trailing r output channels are rotated by the negative query
    angle (rotate-half pairing). A zero angle is the identity; a rotation
    preserves each pair's norm; rotating the result forward again by the same
    angles (the forward formula x cos + rotate_half(x) sin) gives back the
    plain output; and when every value row's rope part is its own rotation
    R_s(v) and the query sits at t, the output only sees s - t: shifting all
    positions by a constant changes nothing."""
    rng = np.random.default_rng(31)
    B, H, N, k, r, D = 2, 3, 40, 16, 16, 64
    x = rng.standard_normal((B, N, D)).astype(np.float32)
    rows = O.quant_rows(O.F32, D, 0, x)
    q = rng.standard_normal((B, H, D)).astype(np.float32)
    idx = np.stack([rng.permutation(N)[:k] for _ in range(B)]).astype(np.int32)
    o0, l0 = O.attention((O.F32, D, 0), D, q, rows, idx, 0.1)
    ang = rng.uniform(-np.pi, np.pi, (B, r // 2))
    cs = np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)
    o1, l1 = O.attention((O.F32, D, 0), D, q, rows, idx, 0.1, rope_cs=cs)
    assert np.array_equal(l0, l1) and np.array_equal(o0[..., :D - r], o1[..., :D - r])
    ident = np.stack([np.ones((B, r // 2)), np.zeros((B, r // 2))], -1).astype(np.float32)
    assert np.array_equal(O.attention((O.F32, D, 0), D, q, rows, idx, 0.1, rope_cs=ident)[0], o0)
    a0, b0 = o0[..., D - r:D - r // 2], o0[..., D - r // 2:]
    a1, b1 = o1[..., D - r:D - r // 2], o1[..., D - r // 2:]
    np.testing.assert_allclose(a1 ** 2 + b1 ** 2, a0 ** 2 + b0 ** 2, rtol=1e-5, atol=1e-7)
    c, s = cs[:, None, :, 0].astype(np.float64), cs[:, None, :, 1].astype(np.float64)
    fwd = np.concatenate([a1 * c - b1 * s, b1 * c + a1 * s], -1)       # x cos + rotate_half(x) sin
    np.testing.assert_allclose(fwd, o0[..., D - r:], rtol=1e-5, atol=1e-6)
    # relative positions only: value rows whose rope part is rotated by their own position s
    freqs = 10000.0 ** (-np.arange(r // 2) / (r // 2))

    def rot(v, pos):                                                  # forward rotation at `pos`
        th = pos[..., None] * freqs
        v1, v2 = v[..., :r // 2], v[..., r // 2:]
        return np.concatenate([v1 * np.cos(th) - v2 * np.sin(th), v2 * np.cos(th) + v1 * np.sin(th)], -1)

    base = rng.standard_normal((B, N, D))
    qz = q.copy()
    qz[..., D - r:] = 0.0                                             # scores independent of the positions
    outs = []
    for shift in (0.0, 37.0):
        pos = np.arange(N, dtype=np.float64)[None].repeat(B, 0) + shift
        xr = base.copy()
        xr[..., D - r:] = rot(base[..., D - r:], pos)
        t = pos[:, -1] + 1.0
        th = t[:, None] * freqs
        cst = np.stack([np.cos(th), np.sin(th)], -1).astype(np.float32)
        outs.append(O.attention((O.F32, D, 0), D, qz, O.quant_rows(O.F32, D, 0, xr.astype(np.float32)), idx, 0.1,
                                rope_cs=cst)[0])
    np.testing.assert_allclose(outs[0], outs[1], rtol=1e-4, atol=1e-5)


def test_bf16_score_topk_matches_the_library_cast_and_lexsort():
    """The bf16-score top-k is the fp32 scores rounded by the library bf16 cast (round to
    nearest even) and ordered by (score desc, position asc): checked on scores full of
    bf16 ties, with masking and k above the visible count."""
    import torch
    rng = np.random.default_rng(21)
    B, N = 3, 5000
    s = (rng.standard_normal((B, N)) * 3).astype(np.float32)
    s[:, ::7] = np.float32(1.0) + np.float32(2.0 ** -9) * rng.integers(0, 3, (B, (N + 6) // 7))  # bf16 midpoints/ties
    nv = np.array([N, 4321, 17], np.int32)
    ref16 = torch.from_numpy(s).to(torch.bfloat16).float().numpy()
    assert np.array_equal(O.bf16_scores(s), ref16)
    for k in (1, 64, 2048, 4400):
        got = O.topk_bf16(s, nv, k)
        for b in range(B):
            n = int(nv[b])
            order = np.lexsort((np.arange(n), -ref16[b, :n].astype(np.float64)))[:min(k, n)]
            assert np.array_equal(np.sort(got[b][got[b] >= 0]), np.sort(order))
            assert np.sum(got[b] < 0) == k - min(k, n)
    # the rounding creates ties that the fp32 order would break: the two selections differ
    assert not np.array_equal(np.sort(O.topk_bf16(s, nv, 64), 1), np.sort(O.topk(s, nv, 64), 1))
