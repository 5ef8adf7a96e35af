"""Python binding of the gfx950 decode hot path (libmla.so, C ABI in include/mla.h).

Argument marshalling only: every function takes torch tensors on the GPU,
checks their dtype / device / layout, and passes raw device pointers and the
current HIP stream to the C entry point of the same name.  All arithmetic runs
in the library's HIP kernels.  There is no fallback: if libmla.so is missing
or fails to load, the functions raise.
"""
import ctypes as C
import os
from typing import NamedTuple, Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla.so")

F32, BF16, E4M3_S128, E2M1_S16, MXFP4, MXFP8 = 0, 1, 2, 3, 4, 5
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "HIP error"}


class Row(NamedTuple):
    """Row format of a cached entry: `dim` channels + `rope` RoPE channels."""
    fmt: int
    dim: int
    rope: int = 0


class _CRow(C.Structure):
    _fields_ = [("dim", C.c_int32), ("rope_dim", C.c_int32), ("fmt", C.c_int32)]


class MLAError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def lib():
    """Load libmla.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "or python sparse_latent_attention_mla_amd/build.py")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
        L.mla_row_bytes.argtypes, L.mla_row_bytes.restype = [_CRow], i64
        L.mla_status_str.argtypes, L.mla_status_str.restype = [i32], C.c_char_p
        L.mla_last_error.argtypes, L.mla_last_error.restype = [], C.c_char_p
        L.mla_version.argtypes, L.mla_version.restype = [], i32
        L.mla_profile_enable.argtypes, L.mla_profile_enable.restype = [i32], i32
        L.mla_profile_read.argtypes = [C.c_char_p, C.POINTER(i32), C.POINTER(C.c_double)]
        L.mla_profile_read.restype = i32
        L.mla_set_option.argtypes, L.mla_set_option.restype = [C.c_char_p, i64], i32
        L.mla_get_option.argtypes, L.mla_get_option.restype = [C.c_char_p, C.POINTER(i64)], i32
        L.mla_last_kernels.argtypes, L.mla_last_kernels.restype = [], C.c_char_p
        L.mla_kv_append_quant.argtypes = [_CRow, _CRow, P, P, P, i32, i32, i64, P, i64, P, i64,
                                          P, P, P, i32, i32, i32, P]
        L.mla_kv_append_quant.restype = i32
        L.mla_indexer_topk_workspace.argtypes, L.mla_indexer_topk_workspace.restype = [i32, i64, i32], sz
        L.mla_compress_append.argtypes = [_CRow, P, P, i32, P, f32, i32, P, P, i32, i64, P, i64, P, P]
        L.mla_compress_append.restype = i32
        L.mla_indexer_topk.argtypes = [_CRow, P, P, f32, P, i64, i64, P, P, i32, i32, i32, i32,
                                       P, P, P, sz, P]
        L.mla_indexer_topk.restype = i32
        L.mla_indexer_topk_bf16.argtypes, L.mla_indexer_topk_bf16.restype = L.mla_indexer_topk.argtypes, i32
        L.mla_append_indexer_topk.argtypes = [_CRow, _CRow, P, P, P, i32, P, i64, P, i64, i64, P, P, P,
                                              i32, i32, i32, P, P, f32, P, i32, i32, i32, P, P, P, sz, P]
        L.mla_append_indexer_topk.restype = i32
        L.mla_append_indexer_topk_bf16.argtypes = L.mla_append_indexer_topk.argtypes
        L.mla_append_indexer_topk_bf16.restype = i32
        L.mla_indexer_pool_workspace.argtypes, L.mla_indexer_pool_workspace.restype = [i32, i64, i32], sz
        L.mla_indexer_pool.argtypes = [P, i64, P, i32, i32, i32, P, P, sz, P]
        L.mla_indexer_pool.restype = i32
        L.mla_sparse_decode_workspace.argtypes = [_CRow, i32, i32, i32, i32, i32, i32]
        L.mla_sparse_decode_workspace.restype = sz
        L.mla_sparse_decode.argtypes = [_CRow, i32, P, P, i64, i64, P, i32, P, P, i32, i32, f32, P, i32, i32,
                                        P, P, P, sz, P]
        L.mla_sparse_decode.restype = i32
        L.mla_sparse_decode_noalloc.argtypes = [_CRow, i32, P, P, i64, i64, P, i32, P, P, i32, i32, f32, P, i32,
                                                i32, P, P, P]
        L.mla_sparse_decode_noalloc.restype = i32
        L.mla_append_sparse_decode.argtypes = [_CRow, i32, P, P, i64, i64, P, i32, P, P, P, P, i32, i32, f32, P, i32,
                                               i32, P, P, P, sz, P]
        L.mla_append_sparse_decode.restype = i32
        L.mla_csa2_group_step.argtypes = [_CRow, _CRow, i32, i32, P, P, P, P, i32, P, i64, P, i64, i64, P, i32, i32,
                                          i32, i32, f32, f32, P, P, i32, i32, i32, i32, i32, P, P, P, P, P, sz, P,
                                          sz, P]
        L.mla_csa2_group_step.restype = i32
        _lib = L
    return _lib


def _crow(r: Row) -> _CRow:
    return _CRow(r.dim, r.rope, r.fmt)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _check(status):
    if status != 0:
        raise MLAError(status, lib().mla_last_error().decode())


def _need(t, name, dtype=None, ndim=None, contiguous=True):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def row_bytes(row: Row) -> int:
    return int(lib().mla_row_bytes(_crow(row)))


def version() -> int:
    return int(lib().mla_version())


def mla_set_option(name: str, value: int) -> None:
    """Force a kernel choice (see include/mla.h); 0 restores the library's own choice."""
    _check(lib().mla_set_option(name.encode(), int(value)))


def mla_get_option(name: str) -> int:
    v = C.c_int64(0)
    _check(lib().mla_get_option(name.encode(), C.byref(v)))
    return int(v.value)


class option:
    """Context manager: set an option for the duration of a block, then restore it."""

    def __init__(self, name: str, value: int):
        self.name, self.value = name, value

    def __enter__(self):
        self.old = mla_get_option(self.name)
        mla_set_option(self.name, self.value)
        return self

    def __exit__(self, *exc):
        mla_set_option(self.name, self.old)
        return False


def mla_last_kernels() -> list:
    """Demangled names of the kernels the calling thread's last compute call launched."""
    s = lib().mla_last_kernels().decode()
    return s.split(";") if s else []


PROFILE_KERNELS = ("kv_append", "indexer_scan", "topk_select", "decode", "decode_merge")


def mla_profile_enable(kernels=()) -> None:
    """Time the named kernels (see PROFILE_KERNELS) from now on; () stops timing."""
    mask = 0
    for name in kernels:
        mask |= 1 << PROFILE_KERNELS.index(name)
    _check(lib().mla_profile_enable(mask))


def mla_profile_read(kernel: str):
    """(launches, total_ms) of `kernel` since the previous read; waits for them to finish.

    Names: "kv_append", "indexer_scan", "topk_select", "decode", "decode_merge".
    """
    n = C.c_int32(0)
    ms = C.c_double(0.0)
    _check(lib().mla_profile_read(kernel.encode(), C.byref(n), C.byref(ms)))
    return int(n.value), float(ms.value)


def query_dtype(row: Row):
    return torch.float32 if row.fmt == F32 else torch.bfloat16


def _cache_stride(cache: Optional[torch.Tensor], name: str) -> int:
    if cache is None:
        return 0
    _need(cache, name, torch.uint8, 3, contiguous=False)
    if cache.stride(2) != 1 or cache.stride(1) != cache.shape[2]:
        raise ValueError(f"{name}: rows must be contiguous [B, capacity, row_bytes]")
    return cache.stride(0)


def _win_ring(win_ring, B, D, name="win_ring"):
    """(format, W) of a window ring: bf16 [B, W, D] or MXFP8 uint8 [B, W, D + D/32]."""
    if win_ring.dtype == torch.uint8:
        _need(win_ring, name, torch.uint8, 3)
        if D % 32 != 0 or win_ring.shape[0] != B or win_ring.shape[2] != D + D // 32:
            raise ValueError(f"{name}: MXFP8 ring [B, W, D + D/32] bytes with D % 32 == 0 expected")
        return MXFP8, win_ring.shape[1]
    _need(win_ring, name, torch.bfloat16, 3)
    if win_ring.shape[0] != B or win_ring.shape[2] != D:
        raise ValueError(f"{name}: bf16 ring [B, W, D] expected")
    return BF16, win_ring.shape[1]


def mla_kv_append_quant(main_row: Row, idx_row: Row, new_main, new_idx, slots,
                        main_cache, idx_cache, new_win=None, win_pos=None, win_ring=None, stream=None):
    """Quantise-append.  new_main fp32 [B, n, D], new_idx fp32 [B, n, d_I], slots int32 [B, n];
    main_cache / idx_cache uint8 [B, capacity, row_bytes] (either may be None);
    new_win fp32 [B, Dw], win_pos int32 [B], win_ring (optional) bf16 [B, W, Dw] or uint8
    [B, W, Dw + Dw/32] for MXFP8 window entries."""
    caches = [c for c in (main_cache, idx_cache) if c is not None]
    capacity = caches[0].shape[1] if caches else 0
    if len(caches) == 2 and main_cache.shape[1] != idx_cache.shape[1]:
        raise ValueError("main and indexer caches must have the same capacity")
    B = n_new = 0
    if caches:
        _need(slots, "slots", torch.int32, 2)
        B, n_new = slots.shape
    if main_cache is not None:
        _need(new_main, "new_main", torch.float32, 3)
        if tuple(new_main.shape) != (B, n_new, main_row.dim + main_row.rope) or main_cache.shape[0] != B:
            raise ValueError("new_main must be [B, n_new, dim + rope] and main_cache [B, capacity, row_bytes]")
        if main_cache.shape[2] != row_bytes(main_row):
            raise ValueError("main_cache rows do not match the row format")
    if idx_cache is not None:
        _need(new_idx, "new_idx", torch.float32, 3)
        if tuple(new_idx.shape) != (B, n_new, idx_row.dim) or idx_cache.shape[0] != B:
            raise ValueError("new_idx must be [B, n_new, idx dim] and idx_cache [B, capacity, row_bytes]")
        if idx_cache.shape[2] != row_bytes(idx_row):
            raise ValueError("idx_cache rows do not match the row format")
    W = Dw = 0
    wfmt = BF16
    if new_win is not None:
        _need(new_win, "new_win", torch.float32, 2)
        _need(win_pos, "win_pos", torch.int32, 1)
        if caches and new_win.shape[0] != B:
            raise ValueError("new_win batch differs from the caches'")
        B, Dw = new_win.shape
        wfmt, W = _win_ring(win_ring, B, Dw)
        if win_pos.shape[0] != B:
            raise ValueError("window shapes: new_win [B, Dw], win_pos [B]")
    _check(lib().mla_kv_append_quant(
        _crow(main_row), _crow(idx_row), _ptr(new_main), _ptr(new_idx), _ptr(slots), B, n_new, capacity,
        _ptr(main_cache), _cache_stride(main_cache, "main_cache"),
        _ptr(idx_cache), _cache_stride(idx_cache, "idx_cache"),
        _ptr(new_win), _ptr(win_pos), _ptr(win_ring), W, Dw, wfmt, _stream(stream)))


def mla_compress_append(main_row: Row, kv, gate, main_cache=None, slots=None, norm_weight=None, eps=1e-6,
                        rope_cs=None, out_entry=None, stream=None):
    """The CSA2 compressor at append: kv, gate fp32 [B, m, D] -> one normalised, gated-pooled entry
    per sequence, quantised into main_cache uint8 [B, capacity, row_bytes] at slots int32 [B] and/or
    returned in out_entry fp32 [B, D]; norm_weight fp32 [D]; rope_cs fp32 [B, r/2, 2]."""
    _need(kv, "kv", torch.float32, 3)
    _need(gate, "gate", torch.float32, 3)
    B, m, D = kv.shape
    if tuple(gate.shape) != (B, m, D) or D != main_row.dim + main_row.rope:
        raise ValueError("kv and gate [B, m, dim + rope] expected")
    capacity = stride = 0
    if main_cache is not None:
        _need(slots, "slots", torch.int32, 1)
        if main_cache.shape[0] != B or main_cache.shape[2] != row_bytes(main_row) or tuple(slots.shape) != (B,):
            raise ValueError("main_cache [B, capacity, row_bytes] and slots [B] expected")
        capacity, stride = main_cache.shape[1], _cache_stride(main_cache, "main_cache")
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", torch.float32, 1)
        if tuple(norm_weight.shape) != (D,):
            raise ValueError("norm_weight [D] expected")
    r = 0
    if rope_cs is not None:
        _need(rope_cs, "rope_cs", torch.float32, 3)
        if rope_cs.shape[0] != B or rope_cs.shape[2] != 2:
            raise ValueError("rope_cs [B, r/2, 2] expected")
        r = 2 * rope_cs.shape[1]
    if out_entry is not None:
        _need(out_entry, "out_entry", torch.float32, 2)
        if tuple(out_entry.shape) != (B, D):
            raise ValueError("out_entry [B, D] expected")
    _check(lib().mla_compress_append(_crow(main_row), _ptr(kv), _ptr(gate), m, _ptr(norm_weight), float(eps), r,
                                     _ptr(rope_cs), _ptr(slots), B, capacity, _ptr(main_cache), stride,
                                     _ptr(out_entry), _stream(stream)))


def mla_indexer_topk_workspace(B: int, capacity: int, k: int) -> int:
    return int(lib().mla_indexer_topk_workspace(B, capacity, k))


def mla_indexer_topk(idx_row: Row, q_idx, w, score_scale: float, idx_cache, n_visible, k: int,
                     out_idx, workspace, out_scores=None, stream=None, cand=None, score_bf16=False):
    """Indexer scan + mask + top-k.  q_idx [B, H_I, d_I] (bf16; fp32 for F32 rows), w fp32 [B, H_I],
    idx_cache uint8 [B, capacity, row_bytes], n_visible int32 [B], out_idx int32 [B, k],
    workspace uint8 of mla_indexer_topk_workspace bytes, zeroed before its first use (every
    successful call leaves it ready for the next), out_scores fp32 [B, capacity] (optional).
    cand: optional int32 [B, n_cand] candidate pool (positions); only those are scored, and
    out_scores is then [B, n_cand].  score_bf16: the bf16-score top-k (mla_indexer_topk_bf16: scores
    rounded to bf16 before they are stored and selected)."""
    _need(q_idx, "q_idx", query_dtype(idx_row), 3)
    _need(w, "w", torch.float32, 2)
    _need(n_visible, "n_visible", torch.int32, 1)
    _need(out_idx, "out_idx", torch.int32, 2)
    _need(workspace, "workspace", torch.uint8)
    stride = _cache_stride(idx_cache, "idx_cache")
    B, H_I, dq = q_idx.shape
    cap = idx_cache.shape[1]
    if dq != idx_row.dim or idx_cache.shape[0] != B or idx_cache.shape[2] != row_bytes(idx_row):
        raise ValueError("q_idx [B, H_I, dim] and idx_cache [B, capacity, row_bytes] must match the row format")
    if tuple(w.shape) != (B, H_I) or tuple(n_visible.shape) != (B,) or tuple(out_idx.shape) != (B, k):
        raise ValueError("w [B, H_I], n_visible [B], out_idx [B, k] expected")
    n_cand = 0
    if cand is not None:
        _need(cand, "cand", torch.int32, 2)
        if cand.shape[0] != B:
            raise ValueError("cand must be [B, n_cand]")
        n_cand = cand.shape[1]
    if out_scores is not None:
        _need(out_scores, "out_scores", torch.float32, 2)
        if tuple(out_scores.shape) != (B, cap if cand is None else n_cand):
            raise ValueError("out_scores must be [B, capacity] ([B, n_cand] with a pool)")
    # an empty pool is still a pool: the C ABI takes it as a non-NULL cand with n_cand 0
    # (never read), so an empty tensor's null data pointer is replaced by out_idx's
    cand_p = None if cand is None else (_ptr(cand) if n_cand > 0 else _ptr(out_idx))
    fn = lib().mla_indexer_topk_bf16 if score_bf16 else lib().mla_indexer_topk
    _check(fn(
        _crow(idx_row), _ptr(q_idx), _ptr(w), float(score_scale), _ptr(idx_cache), stride,
        idx_cache.shape[1], _ptr(n_visible), cand_p, n_cand, B, H_I, k, _ptr(out_idx), _ptr(out_scores),
        _ptr(workspace), workspace.numel(), _stream(stream)))


def mla_indexer_pool_workspace(B: int, capacity: int, block: int = 8) -> int:
    return int(lib().mla_indexer_pool_workspace(B, capacity, block))


def mla_indexer_pool(scores, n_visible, n_blocks: int, out_pos, workspace, block: int = 8, stream=None):
    """Candidate pool of the hierarchical sparse indexer from one layer's scores fp32 [B, capacity]:
    the positions int32 [B, n_blocks * block] of the n_blocks blocks (of `block` consecutive
    positions) with the largest maximum visible score, -1 padded.  workspace: uint8 of
    mla_indexer_pool_workspace bytes, under the zeroing contract of mla_indexer_topk's."""
    _need(scores, "scores", torch.float32, 2)
    _need(n_visible, "n_visible", torch.int32, 1)
    _need(out_pos, "out_pos", torch.int32, 2)
    _need(workspace, "workspace", torch.uint8)
    B, cap = scores.shape
    if tuple(n_visible.shape) != (B,) or tuple(out_pos.shape) != (B, n_blocks * block):
        raise ValueError("n_visible [B] and out_pos [B, n_blocks * block] expected")
    _check(lib().mla_indexer_pool(_ptr(scores), cap, _ptr(n_visible), B, block, n_blocks, _ptr(out_pos),
                                  _ptr(workspace), workspace.numel(), _stream(stream)))


def mla_append_indexer_topk(main_row: Row, idx_row: Row, new_main, new_idx, slots, main_cache, idx_cache,
                            q_idx, w, score_scale: float, n_visible, k: int, out_idx, workspace,
                            new_win=None, win_pos=None, win_ring=None, out_scores=None, stream=None,
                            score_bf16=False):
    """mla_kv_append_quant then mla_indexer_topk in one call (the append rides in the
    scan's launch where the scan kernel can carry it).  Arguments as for those two;
    idx_cache is required, main_cache may be None."""
    if idx_cache is None:
        raise ValueError("idx_cache is required")
    _need(slots, "slots", torch.int32, 2)
    B, n_new = slots.shape
    cap = idx_cache.shape[1]
    if main_cache is not None:
        _need(new_main, "new_main", torch.float32, 3)
        if tuple(new_main.shape) != (B, n_new, main_row.dim + main_row.rope) or tuple(main_cache.shape[:2]) != (B, cap):
            raise ValueError("new_main must be [B, n_new, dim + rope] and main_cache [B, capacity, row_bytes]")
        if main_cache.shape[2] != row_bytes(main_row):
            raise ValueError("main_cache rows do not match the row format")
    _need(new_idx, "new_idx", torch.float32, 3)
    if tuple(new_idx.shape) != (B, n_new, idx_row.dim) or idx_cache.shape[0] != B:
        raise ValueError("new_idx must be [B, n_new, idx dim] and idx_cache [B, capacity, row_bytes]")
    W = Dw = 0
    wfmt = BF16
    if new_win is not None:
        _need(new_win, "new_win", torch.float32, 2)
        _need(win_pos, "win_pos", torch.int32, 1)
        Dw = new_win.shape[1]
        wfmt, W = _win_ring(win_ring, B, Dw)
        if new_win.shape[0] != B or win_pos.shape[0] != B:
            raise ValueError("window shapes: new_win [B, Dw], win_pos [B]")
    _need(q_idx, "q_idx", query_dtype(idx_row), 3)
    _need(w, "w", torch.float32, 2)
    _need(n_visible, "n_visible", torch.int32, 1)
    _need(out_idx, "out_idx", torch.int32, 2)
    _need(workspace, "workspace", torch.uint8)
    _, H_I, dq = q_idx.shape
    if dq != idx_row.dim or q_idx.shape[0] != B or idx_cache.shape[2] != row_bytes(idx_row):
        raise ValueError("q_idx [B, H_I, dim] and idx_cache [B, capacity, row_bytes] must match the row format")
    if tuple(w.shape) != (B, H_I) or tuple(n_visible.shape) != (B,) or tuple(out_idx.shape) != (B, k):
        raise ValueError("w [B, H_I], n_visible [B], out_idx [B, k] expected")
    if out_scores is not None:
        _need(out_scores, "out_scores", torch.float32, 2)
        if tuple(out_scores.shape) != (B, cap):
            raise ValueError("out_scores must be [B, capacity]")
    fn = lib().mla_append_indexer_topk_bf16 if score_bf16 else lib().mla_append_indexer_topk
    _check(fn(
        _crow(main_row), _crow(idx_row), _ptr(new_main), _ptr(new_idx), _ptr(slots), n_new,
        _ptr(main_cache), _cache_stride(main_cache, "main_cache"),
        _ptr(idx_cache), _cache_stride(idx_cache, "idx_cache"), cap,
        _ptr(new_win), _ptr(win_pos), _ptr(win_ring), W, Dw, wfmt,
        _ptr(q_idx), _ptr(w), float(score_scale), _ptr(n_visible), B, H_I, k, _ptr(out_idx), _ptr(out_scores),
        _ptr(workspace), workspace.numel(), _stream(stream)))


def mla_sparse_decode_workspace(main_row: Row, d_v: int, B: int, H: int, k: int, W: int = 0,
                                win_fmt: int = 1) -> int:
    """Workspace bytes of mla_sparse_decode (win_fmt MXFP8 adds the ring's bf16 copy)."""
    return int(lib().mla_sparse_decode_workspace(_crow(main_row), d_v, B, H, k, W, win_fmt))


class _CEpilogue(C.Structure):
    _fields_ = [("sinks", C.c_void_p), ("rope_dim", C.c_int32), ("rope_cs", C.c_void_p)]


def _decode_args(main_row, d_v, q, main_cache, idx, softmax_scale, out, lse, win_ring, win_len, sinks, rope_cs):
    """Checked argument tuple of the decode calls (up to the workspace), and the epilogue struct
    it points to (keep it alive through the call)."""
    _need(q, "q", query_dtype(main_row), 3)
    _need(idx, "idx", torch.int32, 2)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    stride = _cache_stride(main_cache, "main_cache")
    B, H, D = q.shape
    if D != main_row.dim + main_row.rope or main_cache.shape[0] != B or main_cache.shape[2] != row_bytes(main_row):
        raise ValueError("q [B, H, dim + rope] and main_cache [B, capacity, row_bytes] must match the row format")
    if idx.shape[0] != B or tuple(out.shape) != (B, H, d_v) or tuple(lse.shape) != (B, H):
        raise ValueError("idx [B, k], out [B, H, d_v], lse [B, H] expected")
    W = 0
    wfmt = BF16
    if win_ring is not None:
        _need(win_len, "win_len", torch.int32, 1)
        wfmt, W = _win_ring(win_ring, B, D)
        if tuple(win_len.shape) != (B,):
            raise ValueError("win_len [B] expected")
    epi_s, epi = None, None
    if sinks is not None or rope_cs is not None:
        if sinks is not None:
            _need(sinks, "sinks", torch.float32, 1)
            if tuple(sinks.shape) != (H,):
                raise ValueError("sinks [H] expected")
        r = 0
        if rope_cs is not None:
            _need(rope_cs, "rope_cs", torch.float32, 3)
            if rope_cs.shape[0] != B or rope_cs.shape[2] != 2:
                raise ValueError("rope_cs [B, r/2, 2] expected")
            r = 2 * rope_cs.shape[1]
        epi_s = _CEpilogue(None if sinks is None else sinks.data_ptr(), r,
                           None if rope_cs is None else rope_cs.data_ptr())
        epi = C.c_void_p(C.addressof(epi_s))
    args = (_crow(main_row), d_v, _ptr(q), _ptr(main_cache), stride, main_cache.shape[1], _ptr(idx), idx.shape[1],
            _ptr(win_ring), _ptr(win_len), W, wfmt, float(softmax_scale), epi, B, H, _ptr(out), _ptr(lse))
    return args, epi_s


def mla_sparse_decode(main_row: Row, d_v: int, q, main_cache, idx, softmax_scale: float, out, lse,
                      workspace=None, win_ring=None, win_len=None, stream=None, sinks=None, rope_cs=None,
                      new_win=None, win_pos=None):
    """Sparse absorbed-MLA decode.  q [B, H, D] (bf16; fp32 for F32 rows), main_cache uint8
    [B, capacity, row_bytes], idx int32 [B, k], out fp32 [B, H, d_v], lse fp32 [B, H];
    win_ring bf16 [B, W, D] and win_len int32 [B] for the window branch; sinks fp32 [H]
    attention-sink logits (optional); rope_cs fp32 [B, r/2, 2] (cos, sin) un-rotating the
    trailing r output channels (optional). With new_win fp32 [B, D] and win_pos int32 [B]
    the step's window entry is appended to the ring first, in the same call
    (mla_append_sparse_decode)."""
    args, keep = _decode_args(main_row, d_v, q, main_cache, idx, softmax_scale, out, lse, win_ring, win_len, sinks,
                              rope_cs)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    ws = (_ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(stream))
    if new_win is None:
        _check(lib().mla_sparse_decode(*args, *ws))
    else:
        B, D = q.shape[0], q.shape[2]
        if win_ring is None:
            raise ValueError("new_win needs win_ring")
        _need(new_win, "new_win", torch.float32, 2)
        _need(win_pos, "win_pos", torch.int32, 1)
        if tuple(new_win.shape) != (B, D) or tuple(win_pos.shape) != (B,):
            raise ValueError("new_win [B, D] and win_pos [B] expected")
        _check(lib().mla_append_sparse_decode(*args[:8], _ptr(new_win), _ptr(win_pos), *args[8:], *ws))
    del keep


def mla_sparse_decode_noalloc(main_row: Row, d_v: int, q, main_cache, idx, softmax_scale: float, out, lse,
                              win_ring=None, win_len=None, stream=None, sinks=None, rope_cs=None):
    """mla_sparse_decode with the library's static per-GPU scratch instead of a workspace
    (for callers that cannot allocate); calls that overlap on one GPU race."""
    args, keep = _decode_args(main_row, d_v, q, main_cache, idx, softmax_scale, out, lse, win_ring, win_len, sinks,
                              rope_cs)
    _check(lib().mla_sparse_decode_noalloc(*args, _stream(stream)))
    del keep


def csa2_group_step(main_row: Row, idx_row: Row, modes, main_cache, idx_cache, n_visible, k: int,
                    score_scale: float, softmax_scale: float, q, q_idx, w, out, lse, topk_workspace,
                    decode_workspace, idx_out, new_main=None, new_idx=None, slots=None, win_rings=None,
                    new_win=None, win_pos=None, win_len=None, pool=None, score_bf16=False, stream=None,
                    between_layers=None):
    """One decode step of a layer group over one shared cache, as compositions of the
    C-ABI calls ([P1] "DeepSeek-V4.1", "Three modes"; [P4] "CSA2: four layers keep their
    own copy"). modes[l] is "full", "reindex" or "reuse":
      full     the step's append (main row and indexer key, carried in the scan's launch)
               + indexer top-k with the layer's own indexer query + decode;
      reindex  indexer top-k with its own indexer query over the shared indexer keys
               (with `pool`, over the Full layer's candidate pool only) + decode;
      reuse    decode with the latest Full / Reindex layer's indices.
    Every layer attends over the shared main cache with its own query and window.

      q            [L, B, H, D] absorbed queries, one per layer
      q_idx, w     [n, B, H_I, d_I] and [n, B, H_I] for the n Full / Reindex layers, in order
      out, lse     [L, B, H, d_v] and [L, B, H]
      idx_out      list of two int32 [B, k] buffers, used in turn by the selecting layers
      new_main, new_idx, slots   the step's entry (first layer only; new_main None: the main
                   row was appended by other means, e.g. mla_compress_append)
      win_rings    [L, B, W, ...] window rings (bf16 or MXFP8 bytes), new_win [L, B, D] the
                   step's window entries, win_pos [B], win_len [B]; or None (no window)
      pool         None, or (n_blocks, block, full_scores [B, N] fp32, pool_pos int32
                   [B, n_blocks * block]): the Full layer publishes a candidate pool
    The workspaces are one top-k workspace (large enough for the pool too, when used)
    and one decode workspace, each used by one call at a time. between_layers(l), if
    given, is called before layer l > 0 is enqueued (e.g. to time layers apart).
    Returns, per layer, the index tensor it attended."""
    L = len(modes)
    attended, latest, j = [], None, 0
    for l, mode in enumerate(modes):
        if mode not in ("full", "reindex", "reuse"):
            raise ValueError(f"unknown layer mode {mode!r}")
        if l > 0 and between_layers is not None:
            between_layers(l)
        win = (new_win[l], win_pos, win_rings[l]) if win_rings is not None else (None, None, None)
        if mode == "full" or mode == "reindex":
            latest = idx_out[j % 2]
            if l == 0:
                mla_append_indexer_topk(main_row, idx_row, new_main, new_idx, slots,
                                        main_cache if new_main is not None else None, idx_cache, q_idx[j], w[j],
                                        score_scale, n_visible, k, latest, topk_workspace, new_win=win[0],
                                        win_pos=win[1], win_ring=win[2],
                                        out_scores=pool[2] if (pool is not None and mode == "full") else None,
                                        score_bf16=score_bf16, stream=stream)
            else:
                use_pool = pool is not None and mode == "reindex"
                mla_indexer_topk(idx_row, q_idx[j], w[j], score_scale, idx_cache, n_visible, k, latest,
                                 topk_workspace, out_scores=pool[2] if (pool is not None and mode == "full") else None,
                                 cand=pool[3] if use_pool else None, score_bf16=score_bf16, stream=stream)
            if pool is not None and mode == "full":
                mla_indexer_pool(pool[2], n_visible, pool[0], pool[3], topk_workspace, block=pool[1],
                                 stream=stream)
            j += 1
        elif latest is None:
            raise ValueError("a reuse layer needs a preceding full or reindex layer")
        # layers after the first append their window entry in the decode's call
        fused_win = l > 0 and win[0] is not None
        mla_sparse_decode(main_row, out.shape[-1], q[l], main_cache, latest, softmax_scale, out[l], lse[l],
                          decode_workspace, win_rings[l] if win_rings is not None else None,
                          win_len if win_rings is not None else None, stream=stream,
                          new_win=win[0] if fused_win else None, win_pos=win[1] if fused_win else None)
        attended.append(latest)
    return attended


class _CLayer(C.Structure):
    _fields_ = [("mode", C.c_int32), ("q", C.c_void_p), ("q_idx", C.c_void_p), ("w", C.c_void_p),
                ("out", C.c_void_p), ("lse", C.c_void_p), ("win_ring", C.c_void_p), ("new_win", C.c_void_p)]


_LAYER_MODE = {"full": 0, "reindex": 1, "reuse": 2}


def mla_csa2_group_step(main_row: Row, idx_row: Row, modes, main_cache, idx_cache, n_visible, k: int,
                        score_scale: float, softmax_scale: float, q, q_idx, w, out, lse, topk_workspace,
                        decode_workspace, idx_out, new_main=None, new_idx=None, slots=None, win_rings=None,
                        new_win=None, win_pos=None, win_len=None, pool=None, score_bf16=False, stream=None):
    """csa2_group_step as one C call (mla_csa2_group_step): the same layers, kernels and
    results, enqueued back to back from C instead of one Python call per layer and kernel.
    Same arguments as csa2_group_step (every layer's tensors stacked on a leading layer
    axis; q_idx and w one entry per selecting layer, in order); no between_layers. Returns,
    per layer, the index tensor it attended."""
    L = len(modes)
    if L < 1 or any(m not in _LAYER_MODE for m in modes):
        raise ValueError(f"modes must be 'full', 'reindex' or 'reuse', got {modes!r}")
    _need(q, "q", query_dtype(main_row), 4)
    _need(out, "out", torch.float32, 4)
    _need(lse, "lse", torch.float32, 3)
    _need(n_visible, "n_visible", torch.int32, 1)
    _need(topk_workspace, "topk_workspace", torch.uint8)
    _need(decode_workspace, "decode_workspace", torch.uint8)
    if len(idx_out) != 2:
        raise ValueError("idx_out: two int32 [B, k] buffers")
    for i, t in enumerate(idx_out):
        _need(t, f"idx_out[{i}]", torch.int32, 2)
    Lq, B, H, D = q.shape
    n_sel = sum(m != "reuse" for m in modes)
    if Lq != L or out.shape[:3] != (L, B, H) or tuple(lse.shape) != (L, B, H):
        raise ValueError("q [L, B, H, D], out [L, B, H, d_v] and lse [L, B, H] expected")
    if D != main_row.dim + main_row.rope or main_cache.shape[0] != B or main_cache.shape[2] != row_bytes(main_row):
        raise ValueError("q and main_cache must match the main row format")
    if idx_cache.shape[0] != B or idx_cache.shape[2] != row_bytes(idx_row) or idx_cache.shape[1] != main_cache.shape[1]:
        raise ValueError("idx_cache [B, capacity, row_bytes] of the indexer row format, the main cache's capacity")
    _need(q_idx, "q_idx", query_dtype(idx_row), 4)
    _need(w, "w", torch.float32, 3)
    if q_idx.shape[0] < n_sel or w.shape[0] < n_sel or q_idx.shape[1] != B or q_idx.shape[3] != idx_row.dim:
        raise ValueError("q_idx [n, B, H_I, dim] and w [n, B, H_I] for the n selecting layers expected")
    H_I = q_idx.shape[2]
    if tuple(w.shape[1:]) != (B, H_I):
        raise ValueError("w [n, B, H_I] expected")
    n_new = 0
    if new_idx is not None:
        _need(new_idx, "new_idx", torch.float32, 3)
        _need(slots, "slots", torch.int32, 2)
        n_new = slots.shape[1]
        if tuple(slots.shape) != (B, n_new) or tuple(new_idx.shape) != (B, n_new, idx_row.dim):
            raise ValueError("slots [B, n_new] and new_idx [B, n_new, idx dim] expected")
    if new_main is not None:
        _need(new_main, "new_main", torch.float32, 3)
        if tuple(new_main.shape) != (B, n_new, D):
            raise ValueError("new_main [B, n_new, dim + rope] expected")
    W, wfmt = 0, BF16
    if win_rings is not None:
        _need(new_win, "new_win", torch.float32, 3)
        _need(win_pos, "win_pos", torch.int32, 1)
        _need(win_len, "win_len", torch.int32, 1)
        if win_rings.shape[0] != L or tuple(new_win.shape) != (L, B, D):
            raise ValueError("win_rings [L, B, W, ...] and new_win [L, B, dim + rope] expected")
        wfmt, W = _win_ring(win_rings[0], B, D)
    pool_blocks = pool_block = 0
    pool_scores = pool_pos = None
    if pool is not None:
        pool_blocks, pool_block, pool_scores, pool_pos = pool
        _need(pool_scores, "pool scores", torch.float32, 2)
        _need(pool_pos, "pool positions", torch.int32, 2)
    layers = (_CLayer * L)()
    j = 0
    for l, m in enumerate(modes):
        sel = m != "reuse"
        layers[l] = _CLayer(_LAYER_MODE[m], q[l].data_ptr(), q_idx[j].data_ptr() if sel else None,
                            w[j].data_ptr() if sel else None, out[l].data_ptr(), lse[l].data_ptr(),
                            win_rings[l].data_ptr() if W else None, new_win[l].data_ptr() if W else None)
        j += sel
    _check(lib().mla_csa2_group_step(
        _crow(main_row), _crow(idx_row), out.shape[-1], L, C.c_void_p(C.addressof(layers)), _ptr(new_main), _ptr(new_idx), _ptr(slots), n_new,
        _ptr(main_cache), _cache_stride(main_cache, "main_cache"), _ptr(idx_cache),
        _cache_stride(idx_cache, "idx_cache"), idx_cache.shape[1], _ptr(n_visible), B, H, H_I, k,
        float(score_scale), float(softmax_scale), _ptr(win_pos), _ptr(win_len), W, wfmt, int(bool(score_bf16)),
        pool_blocks, pool_block, _ptr(pool_scores), _ptr(pool_pos), _ptr(idx_out[0]), _ptr(idx_out[1]),
        _ptr(topk_workspace), topk_workspace.numel(), _ptr(decode_workspace), decode_workspace.numel(),
        _stream(stream)))
    attended, j = [], 0
    for m in modes:
        if m != "reuse":
            latest = idx_out[j % 2]
            j += 1
        attended.append(latest)
    return attended
