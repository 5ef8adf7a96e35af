"""The sparse decode over bf16 rows when one workgroup serves two head tiles (32
heads) of a split: the launch picks it when one head tile per workgroup would take
more than one round of the CUs. A split streams its rows through LDS in chunks of
64 with the softmax carried online from chunk to chunk, the fewest rows per split
(64 .. 512) that keep one round of workgroups. Against the oracle's attention over
the same rows and index sets, at the spec bar; the test asserts the kernel
that ran."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as WL
from tests import gpu_cases as G

pytestmark = pytest.mark.gpu
C = WL.CONFIGS
CASES = {
    # 3 x 16 splits x 8 head tiles = 384 workgroups of one tile: paired
    "c2p": C["c2"].with_(name="c2p", cid=142, B=3, N=3001),
    # with a 128-entry bf16 window (two extra splits) and a ragged window length
    "c2pw": C["c2"].with_(name="c2pw", cid=143, B=3, N=2500, W=128),
    # no RoPE part: 512-channel rows and window
    "c2p512": C["c2"].with_(name="c2p512", cid=144, B=3, N=2100, rope=0, W=64, softmax_scale=512 ** -0.5),
}


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: GPU tests need an MI355X")


def _decode(case, idx, **kw):
    got_o, got_l = G.gpu_decode(case, 0, idx, **kw)
    launched = G.M.mla_last_kernels()
    assert any("k_decode_pair" in k for k in launched), launched
    return got_o, got_l


@pytest.mark.parametrize("name", sorted(CASES))
def test_paired_decode_matches_the_oracle(name):
    cfg = CASES[name]
    print("paired decode", name, flush=True)
    case = G.build_case(cfg, seed=9)
    rng = np.random.default_rng(cfg.cid)
    B, N, k = cfg.B, cfg.N, cfg.k
    idx = np.stack([rng.permutation(N)[:k] for _ in range(B)]).astype(np.int32)
    idx[1, rng.random(k) < 0.4] = -1                     # ragged: sequence 1 holds fewer rows
    idx[2, -300:] = -1
    if cfg.W:
        case = dataclasses.replace(case, win_len=np.array([cfg.W, 37, 1], np.int32)[:B])
    ref_o, ref_l = G.oracle_attention(case, 0, idx)
    got_o, got_l = _decode(case, idx)
    G.check_attention(got_o, got_l, ref_o, ref_l)
    sinks = (rng.standard_normal(cfg.H) * 3).astype(np.float32)
    ref_o, ref_l = G.oracle_attention(case, 0, idx, sinks=sinks)
    got_o, got_l = _decode(case, idx, sinks=sinks)
    G.check_attention(got_o, got_l, ref_o, ref_l)


def _ragged_idx(rng, N, k, B):
    idx = np.stack([rng.permutation(N)[:k] for _ in range(B)]).astype(np.int32)
    idx[1, rng.random(k) < 0.4] = -1                     # scattered gaps
    idx[2, -300:] = -1                                   # the last splits without a row
    idx[3, :k // 2] = -1                                 # the first half without a row
    idx[4, :] = -1                                       # nothing selected: out = 0, lse = -inf
    return idx


@pytest.mark.parametrize("B,k", [(6, 1000), (16, 2048)])
def test_paired_decode_chunking(B, k):
    """Splits of 128 rows ending in a 40-row chunk (k = 1000: 7 x 128 + 104), and
    splits of 512 rows streamed as 8 chunks (B = 16); sequences whose splits hold
    no row, or only some rows, and one with none selected."""
    cfg = C["c2"].with_(name=f"c2c{B}", cid=160 + B, B=B, N=2300, k=k)
    case = G.build_case(cfg, seed=5)
    rng = np.random.default_rng(B)
    idx = _ragged_idx(rng, cfg.N, k, B)
    ref_o, ref_l = G.oracle_attention(case, 0, idx)
    got_o, got_l = _decode(case, idx)
    G.check_attention(got_o, got_l, ref_o, ref_l)


@pytest.mark.parametrize("H", [32, 64])
def test_paired_decode_head_counts(H):
    """32 and 64 heads: one and two pairs per split (B = 12 and 6 keep more than one
    round of single head tiles)."""
    cfg = C["c2"].with_(name=f"c2h{H}", cid=150 + H, B=12 if H == 32 else 6, N=2300, H=H)
    case = G.build_case(cfg, seed=4)
    rng = np.random.default_rng(H)
    idx = np.stack([rng.permutation(cfg.N)[:cfg.k] for _ in range(cfg.B)]).astype(np.int32)
    idx[:, -7:] = -1
    ref_o, ref_l = G.oracle_attention(case, 0, idx)
    got_o, got_l = _decode(case, idx)
    G.check_attention(got_o, got_l, ref_o, ref_l)
