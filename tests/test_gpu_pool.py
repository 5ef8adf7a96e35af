"""GPU parity of the hierarchical sparse indexer: the candidate pool a Full
layer publishes (mla_indexer_pool) and the Reindex layer's scan and top-k over
that pool (mla_indexer_topk with cand), against the CPU oracle.

Bars:
  * the pool from given scores: exact (integer work on the same floats): the
    same set of blocks, each written as its `block` consecutive positions, the
    same number of -1 blocks;
  * the pool from the oracle's own scores: exact except blocks whose block
    score lies within 1e-4 * max(|theta|, rms) of the n_blocks-th block score;
  * pool scores: |I_gpu - I_ref| <= 1e-4 * max(|I_ref|, rms), -inf for entries
    that are not visible positions;
  * the top-k over a pool: exact except positions whose oracle score lies
    within 1e-4 * max(|theta|, rms) of the k-th visible pool score theta.
"""
import numpy as np
import pytest
import torch

from tests import gpu_cases as G
from tests.test_gpu_parity import case_of, indexer_layers, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


def gpu_pool(scores, n_visible, n_blocks, block, ws=None):
    B, cap = scores.shape
    out = torch.full((B, n_blocks * block), 12345, dtype=torch.int32, device=DEV)
    if ws is None:
        ws = torch.zeros(G.M.mla_indexer_pool_workspace(B, cap, block), dtype=torch.uint8, device=DEV)
    G.M.mla_indexer_pool(G._t(np.asarray(scores, np.float32)), G._t(np.asarray(n_visible, np.int32)), n_blocks,
                         out, ws, block=block)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def pool_blocks(pos, block):
    """Per sequence: (the block indices a pool's positions name, the number of
    -1 blocks), checking that every block slot holds one whole block."""
    B = pos.shape[0]
    runs = pos.reshape(B, -1, block)
    res = []
    for b in range(B):
        r = runs[b]
        pad = r[:, 0] < 0
        assert np.all(r[pad] == -1), "a padding block slot is not all -1"
        first = r[~pad, 0]
        assert np.all(first % block == 0), "a block slot does not start at a block boundary"
        blk = first // block
        assert np.array_equal(r[~pad], blk[:, None] * block + np.arange(block)[None, :]), "not consecutive"
        assert len(np.unique(blk)) == len(blk), "a block is listed twice"
        res.append((blk, int(pad.sum())))
    return res


def check_pool_exact(got_pos, scores, n_visible, n_blocks, block):
    ref = G.O.pool(scores, n_visible, n_blocks, block)
    for b, (blk, npad) in enumerate(pool_blocks(got_pos, block)):
        r = ref[b]
        assert npad == int((r < 0).sum()), f"row {b}: {npad} -1 blocks, oracle {int((r < 0).sum())}"
        assert set(blk.tolist()) == set(r[r >= 0].tolist()), f"row {b}: block sets differ"


def block_scores(scores, nv, block):
    nb = (nv + block - 1) // block
    pad = np.full(nb * block, -np.inf)
    pad[:nv] = scores[:nv]
    return pad.reshape(nb, block).max(axis=1)


def check_pool_near(got_pos, ref_scores, n_visible, n_blocks, block, rel=1e-4):
    """The GPU's pool (from its own scores) against the oracle's scores: block
    membership may differ only for blocks whose oracle block score lies within
    rel * max(|theta|, rms) of the oracle's n_blocks-th block score."""
    n_exempt = 0
    for b, (blk, npad) in enumerate(pool_blocks(got_pos, block)):
        nv = int(n_visible[b])
        bs = block_scores(ref_scores[b].astype(np.float64), nv, block)
        want = min(n_blocks, len(bs))
        assert npad == n_blocks - want
        if want == 0:
            continue
        order = np.lexsort((np.arange(len(bs)), -bs))
        theta = bs[order[want - 1]]
        vis = ref_scores[b, :nv].astype(np.float64)
        rms = np.sqrt(np.mean(vis * vis))
        exempt = np.abs(bs - theta) <= rel * max(abs(theta), rms)
        in_ref = np.zeros(len(bs), bool)
        in_ref[order[:want]] = True
        in_got = np.zeros(len(bs), bool)
        in_got[blk] = True
        bad = (in_ref != in_got) & ~exempt
        assert not bad.any(), f"row {b}: {bad.sum()} non-exempt block differences"
        n_exempt += int(((in_ref != in_got) & exempt).sum())
    return n_exempt


def gpu_topk_pool(case, j, cand, k, n_visible=None, ws=None):
    cfg = case.cfg
    nv = case.n_visible if n_visible is None else n_visible
    B, n_cand = cand.shape
    out_idx = torch.full((B, k), 12345, dtype=torch.int32, device=DEV)
    scores = torch.empty((B, n_cand), dtype=torch.float32, device=DEV)
    if ws is None:
        ws = torch.zeros(G.M.mla_indexer_topk_workspace(B, max(cfg.N, n_cand), k), dtype=torch.uint8,
                         device=DEV)
    G.M.mla_indexer_topk(G.idx_row(cfg), G._qi_gpu(cfg, case.inp.q_idx[j]), G._t(case.inp.w[j]), cfg.sigma,
                         case.g_idx, G._t(nv), k, out_idx, ws, out_scores=scores, cand=G._t(cand))
    torch.cuda.synchronize()
    return out_idx.cpu().numpy(), scores.cpu().numpy()


def check_pool_scores(got, ref, cand, n_visible, rel=1e-4):
    for b in range(ref.shape[0]):
        ok = (cand[b] >= 0) & (cand[b] < n_visible[b])
        assert np.all(np.isneginf(got[b, ~ok])) and np.all(np.isneginf(ref[b, ~ok])), f"row {b}: masked entries"
        if not ok.any():
            continue
        r, g = ref[b, ok].astype(np.float64), got[b, ok].astype(np.float64)
        rms = np.sqrt(np.mean(r * r))
        bound = rel * np.maximum(np.abs(r), rms)
        err = np.abs(g - r)
        assert np.all(err <= bound), f"row {b}: max err {err.max()} vs bound {bound[err.argmax()]}"


def check_pool_topk(got_idx, ref_pool_scores, cand, n_visible, k, rel=1e-4):
    """Set parity over the visible entries of the pool, with the boundary exemption."""
    n_exempt = 0
    for b in range(got_idx.shape[0]):
        ok = (cand[b] >= 0) & (cand[b] < n_visible[b])
        pos = cand[b, ok].astype(np.int64)
        sc = ref_pool_scores[b, ok].astype(np.float64)
        want = min(k, len(pos))
        g = got_idx[b]
        sel = g[g >= 0]
        assert np.sum(g < 0) == k - want, f"row {b}: wrong -1 count"
        assert len(np.unique(sel)) == len(sel), f"row {b}: duplicate positions"
        assert np.all(np.isin(sel, pos)), f"row {b}: a position outside the pool's visible entries"
        if want == 0:
            continue
        order = np.lexsort((pos, -sc))
        theta = sc[order[want - 1]]
        rms = np.sqrt(np.mean(sc * sc))
        exempt = np.abs(sc - theta) <= rel * max(abs(theta), rms)
        in_ref = np.zeros(len(pos), bool)
        in_ref[order[:want]] = True
        in_got = np.isin(pos, sel)
        bad = (in_ref != in_got) & ~exempt
        assert not bad.any(), f"row {b}: {bad.sum()} non-exempt membership differences"
        n_exempt += int(((in_ref != in_got) & exempt).sum())
    return n_exempt


# ---- the pool from given scores ---------------------------------------------
# (B, capacity, n_visible, n_blocks, block): the one-workgroup selection path
# (capacity / block <= 16384) and the many-workgroup one, ragged capacities,
# partial last blocks, more blocks asked for than are visible, empty sequences
POOL_SHAPES = [
    (2, 5003, [5003, 4321], 128, 8),
    (3, 1000, [1000, 37, 0], 100, 8),
    (1, 200003, [199999], 2048, 8),
    (2, 131072, [131072, 90001], 2048, 8),
    (2, 5003, [5003, 4999], 300, 1),
    (2, 70000, [70000, 65536], 64, 64),
    (1, 16, [16], 4, 4),
]


@pytest.mark.parametrize("shape", POOL_SHAPES, ids=lambda s: f"B{s[0]}-cap{s[1]}-nb{s[3]}-blk{s[4]}")
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_pool_exact_on_given_scores(shape, kind):
    B, cap, nv, n_blocks, block = shape
    rng = np.random.default_rng(cap + n_blocks)
    s = rng.standard_normal((B, cap)).astype(np.float32)
    if kind == "ties":                       # few distinct values: block scores tie everywhere
        s = np.round(s, 1).astype(np.float32)
    nv = np.array(nv, np.int32)
    say("pool", shape, kind)
    got = gpu_pool(s, nv, n_blocks, block)
    check_pool_exact(got, s, nv, n_blocks, block)


def test_pool_block_one_is_the_topk_and_all_equal_scores_take_the_first_blocks():
    rng = np.random.default_rng(7)
    s = rng.standard_normal((2, 3000)).astype(np.float32)
    nv = np.array([3000, 2500], np.int32)
    got = gpu_pool(s, nv, 100, 1)
    ref = G.O.topk(s, nv, 100)
    for b in range(2):
        assert set(got[b].tolist()) == set(ref[b].tolist())
    z = np.zeros((1, 4096), np.float32)
    got = gpu_pool(z, np.array([4096], np.int32), 10, 8)
    assert set(got[0].tolist()) == set(range(80))


def test_pool_workspace_shared_with_the_topk():
    """One zeroed workspace, large enough for both, serves pool and top-k calls
    in turn; each leaves the histogram zeroed for the next."""
    case = case_of("c4s")
    cfg = case.cfg
    B, N, k = cfg.B, cfg.N, cfg.k
    size = max(G.M.mla_indexer_topk_workspace(B, N, k), G.M.mla_indexer_pool_workspace(B, N, 8))
    ws = torch.zeros(size, dtype=torch.uint8, device=DEV)
    zero_part = 512 * 128 + B * 8 * (64 + 4096) * 4
    for rep in range(2):
        got_idx, got_s = G.gpu_topk(case, 0, ws=ws)
        assert not bool(ws[:zero_part].any())
        pos = gpu_pool(got_s, case.n_visible, 64, 8, ws=ws)
        assert not bool(ws[:zero_part].any())
        check_pool_exact(pos, got_s, case.n_visible, 64, 8)
        idx2, _ = gpu_topk_pool(case, 0, pos, k, ws=ws)
        assert not bool(ws[:zero_part].any())


# ---- the Reindex layer over a pool -------------------------------------------
@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c4s", "c5s"])
def test_reindex_over_the_full_layers_pool(name):
    """Full layer: GPU scores -> GPU pool (exact against the oracle's pool of
    the same scores, and near the oracle's pool of its own scores); Reindex
    layer: its own query over the pool's positions, scores and top-k against
    the oracle on the same pool (and the Full layer's query re-ranked inside
    its own pool)."""
    case = case_of(name)
    cfg = case.cfg
    nv = case.n_visible
    n_blocks = max(1, min(2048, cfg.N // 32))
    block = 8
    got_idx, got_s = G.gpu_topk(case, 0)
    ref_s = G.oracle_scores(case, 0)
    pos = gpu_pool(got_s, nv, n_blocks, block)
    check_pool_exact(pos, got_s, nv, n_blocks, block)
    ne = check_pool_near(pos, ref_s, nv, n_blocks, block)
    say("pool", name, "blocks", n_blocks, "exempt block swaps", ne)
    layers = indexer_layers(cfg)
    j = layers[1][1] if len(layers) > 1 else 0
    for jj in sorted({0, j}):
        k = min(cfg.k, n_blocks)
        idx_p, sc_p = gpu_topk_pool(case, jj, pos, k)
        ref_p = G.oracle_scores(case, jj, cand=pos)
        check_pool_scores(sc_p, ref_p, pos, nv)
        check_pool_topk(idx_p, ref_p, pos, nv, k)


@pytest.mark.parametrize("name", ["c1", "c2s", "c3s", "c4s", "c4xs"])
def test_topk_over_arbitrary_pools(name):
    """Pools that are not block runs: shuffled distinct positions mixed with
    -1, other negatives, positions past n_visible and past the capacity; sizes
    that are not tile multiples; k above and below the number of visible
    entries; an empty pool."""
    case = case_of(name)
    cfg = case.cfg
    B, N = cfg.B, cfg.N
    rng = np.random.default_rng(cfg.cid)
    nv = np.array([N] + [max(1, N // 3)] * (B - 1), np.int32)
    for n_cand, k in ((1000, 37), (777, cfg.k), (3, 5), (0, 4)):
        n_cand = min(n_cand, N + 50)
        cand = np.empty((B, n_cand), np.int32)
        for b in range(B):
            c = rng.permutation(N + 50)[:n_cand].astype(np.int64)
            c[rng.random(n_cand) < 0.05] = -1
            c[rng.random(n_cand) < 0.02] = -7
            cand[b] = c
        say("arbitrary pool", name, n_cand, k)
        idx_p, sc_p = gpu_topk_pool(case, 0, cand, k, n_visible=nv)
        ref_p = G.oracle_scores(case, 0, n_visible=nv, cand=cand)
        check_pool_scores(sc_p, ref_p, cand, nv)
        check_pool_topk(idx_p, ref_p, cand, nv, k)


def test_c5_full_size_pool_and_reindex():
    """V4.1 sizes: 524,288 entries, a 2,048-block pool of 16,384 positions, and
    the Reindex layer's top-512 inside it."""
    case = case_of("c5")
    cfg = case.cfg
    nv = case.n_visible
    got_idx, got_s = G.gpu_topk(case, 0)
    say("c5 full: pool")
    pos = gpu_pool(got_s, nv, 2048, 8)
    check_pool_exact(pos, got_s, nv, 2048, 8)
    ref_s = G.oracle_scores(case, 0)
    ne = check_pool_near(pos, ref_s, nv, 2048, 8)
    say("c5 full: exempt block swaps", ne)
    say("c5 full: reindex over the pool")
    idx_p, sc_p = gpu_topk_pool(case, 1, pos, cfg.k)
    ref_p = G.oracle_scores(case, 1, cand=pos)
    check_pool_scores(sc_p, ref_p, pos, nv)
    ne = check_pool_topk(idx_p, ref_p, pos, nv, cfg.k)
    say("c5 full: exempt boundary swaps", ne)
