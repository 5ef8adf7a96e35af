"""Python view of the CPU oracle (oracle/oracle.c) on numpy arrays.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  It shares no
code with the HIP library.

Formats: 0 = F32, 1 = BF16, 2 = E4M3 with one fp32 scale per 128 channels
(plus bf16 RoPE tail), 3 = E2M1 with one E4M3 scale per 16 channels.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

F32, BF16, E4M3_S128, E2M1_S16, MXFP4, MXFP8 = 0, 1, 2, 3, 4, 5

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        P = C.c_void_p
        i32, i64, f32 = C.c_int32, C.c_int64, C.c_float
        L.orc_e4m3_value.argtypes, L.orc_e4m3_value.restype = [C.c_uint32], C.c_double
        L.orc_e8m0_value.argtypes, L.orc_e8m0_value.restype = [C.c_uint32], C.c_double
        L.orc_mx_scale.argtypes, L.orc_mx_scale.restype = [C.c_float], C.c_uint32
        L.orc_mx8_scale.argtypes, L.orc_mx8_scale.restype = [C.c_float], C.c_uint32
        L.orc_e4m3_encode.argtypes, L.orc_e4m3_encode.restype = [f32], C.c_uint32
        L.orc_e2m1_value.argtypes, L.orc_e2m1_value.restype = [C.c_uint32], C.c_double
        L.orc_e2m1_encode.argtypes, L.orc_e2m1_encode.restype = [f32], C.c_uint32
        L.orc_bf16_encode.argtypes, L.orc_bf16_encode.restype = [f32], C.c_uint32
        L.orc_bf16_value.argtypes, L.orc_bf16_value.restype = [C.c_uint32], f32
        for n in ("orc_e4m3_encode_n", "orc_e2m1_encode_n", "orc_bf16_encode_n"):
            getattr(L, n).argtypes, getattr(L, n).restype = [P, i64, P], None
        L.orc_row_bytes.argtypes, L.orc_row_bytes.restype = [i32, i32, i32], i64
        L.orc_quant_row.argtypes, L.orc_quant_row.restype = [i32, i32, i32, P, P], i32
        L.orc_dequant_row.argtypes, L.orc_dequant_row.restype = [i32, i32, i32, P, P], i32
        L.orc_append.argtypes = [i32, i32, i32, i32, i32, P, P, P, i32, i32, i64,
                                 P, i64, P, i64, P, P, P, i32, i32]
        L.orc_append.restype = i32
        L.orc_indexer_scores.argtypes = [i32, i32, P, P, f32, P, i64, P, P, i32, i32, i32, i64, P]
        L.orc_indexer_scores.restype = i32
        L.orc_topk.argtypes, L.orc_topk.restype = [P, i64, P, P, i32, i32, i32, P], i32
        L.orc_pool.argtypes, L.orc_pool.restype = [P, i64, P, i32, i32, i32, P], i32
        L.orc_attention.argtypes = [i32, i32, i32, i32, P, P, i64, i64, P, i32, P, P, i32,
                                    f32, P, i32, P, i32, i32, P, P]
        L.orc_attention.restype = i32
        L.orc_num_threads.argtypes, L.orc_num_threads.restype = [], i32
        L.orc_set_threads.argtypes, L.orc_set_threads.restype = [i32], None
        L.orc_compress.argtypes = [i32, i32, P, P, P, C.c_double, i32, P, i32, P]
        L.orc_compress.restype = i32
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (code {rc})")


def set_num_threads(n: int) -> None:
    """Threads the oracle's parallel loops use from now on (timing only)."""
    lib().orc_set_threads(int(n))


def num_threads() -> int:
    return int(lib().orc_num_threads())


# ---- scalar codecs (vectorised over numpy arrays) ------------------------
def e4m3_value(codes):
    codes = np.asarray(codes, dtype=np.uint32)
    return np.array([lib().orc_e4m3_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def e8m0_value(codes):
    codes = np.asarray(codes, dtype=np.uint32)
    return np.array([lib().orc_e8m0_value(int(c)) for c in codes.ravel()]).reshape(codes.shape)


def mx_scale(amax):
    """The E8M0 code of an MXFP4 block whose largest magnitude is amax (fp32)."""
    return int(lib().orc_mx_scale(float(np.float32(amax))))


def mx8_scale(amax):
    """The E8M0 code of an MXFP8 (E4M3) block whose largest magnitude is amax (fp32)."""
    return int(lib().orc_mx8_scale(float(np.float32(amax))))


def e2m1_value(nibs):
    nibs = np.asarray(nibs, dtype=np.uint32)
    return np.array([lib().orc_e2m1_value(int(c)) for c in nibs.ravel()]).reshape(nibs.shape)


def _enc_n(fn, x, dt):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=dt)
    getattr(lib(), fn)(_p(x), x.size, _p(out))
    return out


def e4m3_encode(x):
    return _enc_n("orc_e4m3_encode_n", x, np.uint8)


def e2m1_encode(x):
    return _enc_n("orc_e2m1_encode_n", x, np.uint8)


def bf16_encode(x):
    return _enc_n("orc_bf16_encode_n", x, np.uint16)


def bf16_value(h):
    h = np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16
    return h.view(np.float32)


# ---- rows ----------------------------------------------------------------
def row_bytes(fmt, dim, rope=0) -> int:
    return int(lib().orc_row_bytes(fmt, dim, rope))


def quant_rows(fmt, dim, rope, x):
    """x: [..., dim+rope] fp32 -> uint8 [..., row_bytes]."""
    x = _c(x, np.float32)
    rb = row_bytes(fmt, dim, rope)
    if rb < 0 or x.shape[-1] != dim + rope:
        raise ValueError("bad row format or width")
    flat = x.reshape(-1, dim + rope)
    out = np.empty((flat.shape[0], rb), dtype=np.uint8)
    L = lib()
    for i in range(flat.shape[0]):
        _check(L.orc_quant_row(fmt, dim, rope, _p(flat[i]), _p(out[i])), "quant_row")
    return out.reshape(x.shape[:-1] + (rb,))


def dequant_rows(fmt, dim, rope, rows):
    """uint8 [..., row_bytes] -> exact float64 values [..., dim+rope]."""
    rows = _c(rows, np.uint8)
    rb = row_bytes(fmt, dim, rope)
    flat = rows.reshape(-1, rb)
    out = np.empty((flat.shape[0], dim + rope), dtype=np.float64)
    L = lib()
    for i in range(flat.shape[0]):
        _check(L.orc_dequant_row(fmt, dim, rope, _p(flat[i]), _p(out[i])), "dequant_row")
    return out.reshape(rows.shape[:-1] + (dim + rope,))


# ---- the path ------------------------------------------------------------
def append(main_row, idx_row, new_main, new_idx, slots, main_cache, idx_cache,
           new_win=None, win_pos=None, win_ring=None):
    """In-place append into numpy caches.  main_row / idx_row: (fmt, dim, rope).

    main_cache: uint8 [B, capacity, row_bytes] (or None); idx_cache likewise;
    win_ring: uint16 [B, W, Dw] bf16 bits (or None)."""
    B, n_new = slots.shape
    mf, md, mr = main_row
    jf, jd, _ = idx_row
    cap = (main_cache if main_cache is not None else idx_cache).shape[1] if (
        main_cache is not None or idx_cache is not None) else 0
    W = Dw = 0
    if win_ring is not None:
        _, W, Dw = win_ring.shape
    for a in (main_cache, idx_cache, win_ring):
        if a is not None and not a.flags.c_contiguous:
            raise ValueError("caches must be C-contiguous")
    rc = lib().orc_append(
        mf, md, mr, jf, jd, _p(_c(new_main, np.float32)), _p(_c(new_idx, np.float32)),
        _p(_c(slots, np.int32)), B, n_new, cap,
        _p(main_cache), 0 if main_cache is None else main_cache.strides[0],
        _p(idx_cache), 0 if idx_cache is None else idx_cache.strides[0],
        _p(_c(new_win, np.float32)), _p(_c(win_pos, np.int32)), _p(win_ring), W, Dw)
    _check(rc, "append")


def indexer_scores(idx_row, q_idx, w, sigma, idx_cache, n_visible, cand=None):
    """q_idx: [B, H_I, d_I] (exact values of the bf16 inputs); w: [B, H_I];
    idx_cache: uint8 [B, N, row_bytes].  Returns fp32 [B, N] (or [B, n_cand])."""
    fmt, dim, _ = idx_row
    q_idx = _c(q_idx, np.float32)
    B, H_I, d = q_idx.shape
    if d != dim:
        raise ValueError("q_idx width")
    idx_cache = _c(idx_cache, np.uint8)
    N = idx_cache.shape[1]
    cand_a = _c(cand, np.int32)
    n_out = N if cand is None else cand_a.shape[1]
    out = np.empty((B, n_out), dtype=np.float32)
    rc = lib().orc_indexer_scores(fmt, dim, _p(q_idx), _p(_c(w, np.float32)), float(sigma),
                                  _p(idx_cache), idx_cache.strides[0],
                                  _p(_c(n_visible, np.int32)), _p(cand_a),
                                  0 if cand is None else n_out, B, H_I, N, _p(out))
    _check(rc, "indexer_scores")
    return out


def topk(scores, n_visible, k, n_rows=None, cand=None):
    scores = _c(scores, np.float32)
    B = scores.shape[0]
    n_rows = scores.shape[1] if n_rows is None else n_rows
    cand_a = _c(cand, np.int32)
    out = np.empty((B, k), dtype=np.int32)
    rc = lib().orc_topk(_p(scores), n_rows, _p(_c(n_visible, np.int32)), _p(cand_a),
                        0 if cand is None else cand_a.shape[1], B, k, _p(out))
    _check(rc, "topk")
    return out


def bf16_scores(scores):
    """Index scores as the bf16-score top-k keeps them ([P1] "DeepSeek-V4", "The indexer in
    four bits": scores in bf16 instead of fp32): each fp32 score rounded to the nearest bf16
    value, ties to even (-inf stays -inf), returned as fp32 values."""
    s = _c(scores, np.float32)
    return bf16_value(bf16_encode(s)).reshape(s.shape)


def topk_bf16(scores, n_visible, k, cand=None):
    """The bf16-score top-k: the selection of topk() over bf16_scores(scores) -- the k visible
    rows of largest bf16 score, ties going to the smaller position."""
    return topk(bf16_scores(scores), n_visible, k, cand=cand)


def pool(scores, n_visible, n_blocks, block=8):
    """Candidate pool of the hierarchical sparse indexer: the block indices
    [B, n_blocks] of the n_blocks blocks (of `block` consecutive positions) with
    the largest maximum visible score, -1 padded."""
    scores = _c(scores, np.float32)
    B, n_rows = scores.shape
    out = np.empty((B, n_blocks), dtype=np.int32)
    rc = lib().orc_pool(_p(scores), n_rows, _p(_c(n_visible, np.int32)), B, block, n_blocks, _p(out))
    _check(rc, "pool")
    return out


def pool_positions(blocks, block=8):
    """The positions [B, block * n_blocks] of a pool's blocks (-1 for -1)."""
    blocks = np.asarray(blocks, np.int64)
    pos = blocks[:, :, None] * block + np.arange(block)[None, None, :]
    pos = np.where(blocks[:, :, None] < 0, -1, pos)
    return pos.reshape(blocks.shape[0], -1).astype(np.int32)


def attention(main_row, d_v, q, main_cache, idx, softmax_scale, win_ring=None, win_len=None, sinks=None,
              rope_cs=None):
    """q: [B, H, dim+rope] (exact values of the bf16 inputs); main_cache uint8
    [B, capacity, row_bytes]; idx int32 [B, k]; win_ring uint16 [B, W, dim+rope];
    sinks: optional fp32 [H] attention-sink logits; rope_cs: optional fp32 [B, r/2, 2]
    (cos, sin) un-rotating the trailing r output channels.  Returns (out fp32 [B, H, d_v], lse fp32 [B, H])."""
    fmt, dim, rope = main_row
    q = _c(q, np.float32)
    B, H, D = q.shape
    if D != dim + rope:
        raise ValueError("q width")
    main_cache = _c(main_cache, np.uint8)
    idx = _c(idx, np.int32)
    k = idx.shape[1]
    W = 0
    if win_ring is not None:
        win_ring = _c(win_ring, np.uint16)
        W = win_ring.shape[1]
    out = np.empty((B, H, d_v), dtype=np.float32)
    lse = np.empty((B, H), dtype=np.float32)
    rc = lib().orc_attention(fmt, dim, rope, d_v, _p(q), _p(main_cache), main_cache.strides[0],
                             main_cache.shape[1], _p(idx), k, _p(win_ring),
                             _p(_c(win_len, np.int32)), W, float(softmax_scale), _p(_c(sinks, np.float32)),
                             0 if rope_cs is None else 2 * np.asarray(rope_cs).shape[1],
                             _p(_c(rope_cs, np.float32)), B, H, _p(out), _p(lse))
    _check(rc, "attention")
    return out, lse


def compress(kv, gate, norm_weight=None, eps=1e-6, rope_cs=None):
    """The CSA2 compressor: kv, gate fp32 [B, m, D] -> normalised, gated-pooled entries fp32 [B, D]
    (rope_cs [B, r/2, 2] rotates the trailing r channels forward)."""
    kv = _c(kv, np.float32)
    gate = _c(gate, np.float32)
    B, m, D = kv.shape
    g = None if norm_weight is None else _c(norm_weight, np.float32)
    cs = None if rope_cs is None else _c(rope_cs, np.float32)
    r = 0 if cs is None else 2 * cs.shape[1]
    out = np.empty((B, D), dtype=np.float32)
    rc = lib().orc_compress(D, m, _p(kv), _p(gate), _p(g), float(eps), r, _p(cs), B, _p(out))
    if rc != 0:
        raise ValueError(f"orc_compress failed ({rc})")
    return out
