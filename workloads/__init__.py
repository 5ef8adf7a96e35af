"""Synthetic decode workloads: shapes of the five configurations and seeded inputs.

This module holds no arithmetic of the attention method.  It only defines the
shapes and draws i.i.d. N(0, 1) fp32 tensors from a counter-based generator
(SplitMix64 + Box-Muller, see gen.c), so that the oracle side and the GPU side
are fed the same inputs.  Both sides import it; it imports neither.

Recipe of one decode step (shared by tests and the benchmark):
  * the cache holds the entries of all earlier positions; the step appends the
    entry of the current position and queries it, so every row is visible;
  * main entries, indexer keys, queries, indexer queries, indexer weights and
    window entries are independent N(0, 1) draws (tensor ids below);
    indexer weights are then multiplied by H_I ** -0.5 and queries are rounded
    to bf16 by the caller (fp32 kept for the fp32 configuration);
  * with pooling ratio m = 2 the tokens are drawn and consecutive pairs are
    averaged in fp32 ((a + b) * 0.5) to form one entry (a stand-in for the
    learned compressor, which needs trained weights).
"""
import ctypes as C
import dataclasses
import math
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libsynth.so")

# tensor ids of the generator streams
T_MAIN, T_IDX, T_Q, T_QIDX, T_W, T_WIN = 1, 2, 3, 4, 5, 6
T_GATE = 7            # gate logits of the CSA2 compressor's tokens

# row formats (numbering used by the library and the oracle alike)
F32, BF16, E4M3_S128, E2M1_S16, MXFP4, MXFP8 = 0, 1, 2, 3, 4, 5


def build(verbose=False):
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           os.path.join(HERE, "gen.c"), "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = C.CDLL(LIB)
        L.syn_splitmix64.argtypes, L.syn_splitmix64.restype = [C.c_uint64, C.c_uint64], C.c_uint64
        L.syn_stream_key.argtypes = [C.c_uint64, C.c_uint64, C.c_uint64]
        L.syn_stream_key.restype = C.c_uint64
        L.syn_normal_f32.argtypes = [C.c_uint64, C.c_uint64, C.c_int64, C.c_void_p]
        L.syn_normal_f32.restype = None
        _lib = L
    return _lib


def splitmix64(key: int, n: int) -> int:
    return int(_L().syn_splitmix64(key, n))


def normal(seed: int, config_id: int, tensor_id: int, shape, offset: int = 0) -> np.ndarray:
    """Elements [offset, offset + prod(shape)) of the N(0,1) stream, fp32."""
    key = _L().syn_stream_key(seed, config_id, tensor_id)
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.float32)
    if n:
        _L().syn_normal_f32(key, offset, n, out.ctypes.data_as(C.c_void_p))
    return out.reshape(shape)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return it as fp32 values.
    Input preparation only (queries are handed to both sides in bf16)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    return r.view(np.float32).reshape(np.shape(x))


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cid: int              # generator config id
    B: int                # sequences
    N: int                # visible cache rows per sequence at the decode step
    H: int                # query heads
    dim: int              # latent channels of a main row (K = [latent; rope])
    rope: int             # RoPE channels of a main row stored separately
    d_v: int              # value width (leading channels of the row)
    H_I: int              # indexer heads
    d_I: int              # indexer head dim
    k: int                # top-k
    main_fmt: int
    idx_fmt: int
    W: int = 0            # window entries (0: no window branch)
    m: int = 1            # tokens pooled per entry
    layers: tuple = ("full",)   # CSA2 modes of the layer group
    softmax_scale: float = 0.0
    desc: str = ""

    @property
    def D(self):
        return self.dim + self.rope

    @property
    def sigma(self):
        return self.d_I ** -0.5

    @property
    def w_scale(self):
        return self.H_I ** -0.5

    @property
    def tokens(self):
        return self.N * self.m

    def with_(self, **kw):
        return dataclasses.replace(self, **kw)


CONFIGS = {
    "c1": Config("c1", 1, B=1, N=256, H=16, dim=64, rope=16, d_v=64, H_I=4, d_I=32, k=32,
                 main_fmt=F32, idx_fmt=F32, softmax_scale=80 ** -0.5,
                 desc="tiny fp32 case: B=1, T=256, 16 heads, latent 64 + rope 16, "
                      "indexer 4x32, top-32"),
    "c2": Config("c2", 2, B=8, N=8192, H=128, dim=512, rope=64, d_v=512, H_I=64, d_I=128,
                 k=2048, main_fmt=BF16, idx_fmt=BF16, softmax_scale=192 ** -0.5,
                 desc="V3.2-shaped decode, bf16 cache: B=8, T=8192, 128 heads, 576/512, "
                      "indexer 64x128, top-2048"),
    "c3": Config("c3", 3, B=4, N=131072, H=128, dim=512, rope=64, d_v=512, H_I=64, d_I=128,
                 k=2048, main_fmt=E4M3_S128, idx_fmt=E4M3_S128, softmax_scale=192 ** -0.5,
                 desc="V3.2-shaped decode, E4M3 caches (656 B / 132 B rows): B=4, T=131072, "
                      "128 heads, indexer 64x128, top-2048"),
    "c4": Config("c4", 4, B=4, N=262144, H=64, dim=512, rope=0, d_v=512, H_I=64, d_I=128,
                 k=512, main_fmt=E2M1_S16, idx_fmt=E2M1_S16, W=128, softmax_scale=512 ** -0.5,
                 desc="V4.1-Flash format, one Full layer: B=4, T=262144, FP4 rows (288 B / 72 B), "
                      "64 heads x 512, indexer 64x128, top-512, 128-entry bf16 window"),
    "c4x": Config("c4x", 6, B=4, N=262144, H=64, dim=512, rope=0, d_v=512, H_I=64, d_I=128,
                  k=512, main_fmt=E2M1_S16, idx_fmt=MXFP4, W=128, softmax_scale=512 ** -0.5,
                  desc="c4 with V4's MXFP4 indexer: B=4, T=262144, FP4 main rows (288 B), MXFP4 "
                       "indexer keys (68 B) and FP4 query-key products, 64 heads x 512, indexer 64x128, "
                       "top-512, 128-entry bf16 window"),
    "c5": Config("c5", 5, B=1, N=524288, H=64, dim=512, rope=0, d_v=512, H_I=64, d_I=128,
                 k=512, main_fmt=E2M1_S16, idx_fmt=E2M1_S16, W=128, m=2,
                 layers=("full", "reindex", "reuse", "reuse", "reuse", "reuse"),
                 softmax_scale=512 ** -0.5,
                 desc="V4.1-style CSA2 group: 1,048,576 tokens pooled 2:1 into 524,288 FP4 "
                      "entries, Full + Reindex + 4 Reuse layers, 64 heads, top-512, "
                      "128-entry bf16 window per layer"),
}


@dataclasses.dataclass
class StepInputs:
    """fp32 inputs of one decode step (layer group) of a configuration."""
    cfg: Config
    main: np.ndarray      # [B, N, D]   entry vectors of positions 0..N-1 (last one is appended);
                          #             None when m > 1 (pooled by the compressor, see compressor_tokens)
    idx: np.ndarray       # [B, N, d_I] indexer keys
    q: np.ndarray         # [L, B, H, D]      (bf16-rounded unless fp32 config)
    q_idx: np.ndarray     # [L_I, B, H_I, d_I] (bf16-rounded unless fp32 config)
    w: np.ndarray         # [L_I, B, H_I]     (already x H_I^-0.5)
    win: np.ndarray       # [L, B, W, D] window entries of positions p-W+1..p (or None)

    @property
    def n_visible(self):
        return np.full((self.cfg.B,), self.cfg.N, dtype=np.int32)


def n_indexers(cfg: Config) -> int:
    return sum(1 for m in cfg.layers if m in ("full", "reindex"))


def step_inputs(cfg: Config, seed: int = 0) -> StepInputs:
    B, N, D, L = cfg.B, cfg.N, cfg.D, len(cfg.layers)
    LI = n_indexers(cfg)
    cid = cfg.cid
    # with m > 1 tokens per entry the main entries come from the CSA2 compressor over
    # compressor_tokens(); the caller pools them (main is None here)
    main = normal(seed, cid, T_MAIN, (B, N, D)) if cfg.m == 1 else None
    idx = normal(seed, cid, T_IDX, (B, N, cfg.d_I))
    lowp = cfg.main_fmt != F32
    q = normal(seed, cid, T_Q, (L, B, cfg.H, D))
    q_idx = normal(seed, cid, T_QIDX, (LI, B, cfg.H_I, cfg.d_I))
    if lowp:
        q = bf16_round(q)
        q_idx = bf16_round(q_idx)
    w = normal(seed, cid, T_W, (LI, B, cfg.H_I)) * np.float32(cfg.w_scale)
    win = normal(seed, cid, T_WIN, (L, B, cfg.W, D)) if cfg.W else None
    return StepInputs(cfg, main, idx, q, q_idx, w.astype(np.float32), win)


def compressor_tokens(cfg: Config, seed: int, b: int, n0: int, n1: int, tensor_offset: int = 0):
    """The compressor inputs of entries n0 .. n1-1 of sequence b: kv and gate logits fp32
    [n1 - n0, m, D], i.i.d. N(0, 1), m tokens per entry."""
    D, m, N = cfg.D, cfg.m, cfg.N
    off = (b * N + n0) * m * D
    kv = normal(seed, cfg.cid, T_MAIN + tensor_offset, (n1 - n0, m, D), offset=off)
    gate = normal(seed, cfg.cid, T_GATE + tensor_offset, (n1 - n0, m, D), offset=off)
    return kv, gate


def window_entry_bytes(cfg: Config, win_fmt: int = BF16) -> int:
    """Bytes of one window entry: bf16, or MXFP8 (E4M3 codes + one E8M0 byte per 32 channels)."""
    return cfg.D + cfg.D // 32 if win_fmt == MXFP8 else 2 * cfg.D


def algorithmic_bytes(cfg: Config, pool_blocks: int = 0, block: int = 8, win_fmt: int = BF16) -> dict:
    """Bytes one decode step (layer group) must move, by part.  Materialised
    scores and split-K partials are excluded: they are implementation traffic.
    With pool_blocks > 0 the first indexer layer publishes a candidate pool of
    that many blocks (hierarchical sparse indexer): the later indexer layers
    read only the pool's rows, and the pool's positions are written once and
    read by each of them."""
    rb_main = _row_bytes(cfg.main_fmt, cfg.dim, cfg.rope)
    rb_idx = _row_bytes(cfg.idx_fmt, cfg.d_I, 0)
    qb = 4 if cfg.main_fmt == F32 else 2
    B, L, LI = cfg.B, len(cfg.layers), n_indexers(cfg)
    k_eff = min(cfg.k, cfg.N)
    pool_rows = min(pool_blocks * block, cfg.N) if pool_blocks else cfg.N
    parts = {
        "scan": B * cfg.N * rb_idx + (LI - 1) * B * pool_rows * rb_idx,
        "q_idx_w": LI * B * cfg.H_I * (cfg.d_I * qb + 4),
        "indices": LI * B * cfg.k * 4 + L * B * cfg.k * 4,
        "gather": L * B * k_eff * rb_main,
        "window": L * B * cfg.W * window_entry_bytes(cfg, win_fmt),
        "q": L * B * cfg.H * cfg.D * qb,
        "out": L * B * cfg.H * (cfg.d_v + 1) * 4,
        "append": B * (rb_main + rb_idx + 4 * (cfg.D + cfg.d_I)) + L * B * (4 * cfg.D + window_entry_bytes(cfg, win_fmt)) * (cfg.W > 0),
    }
    if pool_blocks and LI > 1:
        parts["pool"] = B * pool_blocks * block * 4 * LI
    parts["total"] = sum(parts.values())
    return parts


def _row_bytes(fmt, dim, rope):
    if fmt == F32:
        return 4 * (dim + rope)
    if fmt == BF16:
        return 2 * (dim + rope)
    if fmt == E4M3_S128:
        return dim + 4 * (dim // 128) + 2 * rope
    if fmt == E2M1_S16:
        return dim // 2 + dim // 16
    if fmt == MXFP4:
        return dim // 2 + dim // 32
    raise ValueError(fmt)
