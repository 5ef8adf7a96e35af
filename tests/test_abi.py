"""The C ABI library loads and exports every entry point include/mla.h declares,
and host-side validation rejects bad arguments before any launch.  CPU only:
no call here reaches the GPU."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def M():
    import sparse_latent_attention_mla_amd as M
    if not os.path.exists(M.LIB_PATH):
        pytest.fail("libmla.so is not built (run __graft_entry__.build())")
    return M


def test_header_declares_the_three_path_calls():
    names = declared_functions()
    for n in ("mla_kv_append_quant", "mla_indexer_topk", "mla_sparse_decode", "mla_append_indexer_topk", "mla_compress_append",
              "mla_indexer_pool", "mla_compress_append"):
        assert n in names


def test_library_exports_every_declared_symbol(M):
    lib = C.CDLL(M.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"


def test_row_bytes_and_status_strings(M):
    R = M.Row
    assert M.row_bytes(R(M.E4M3_S128, 512, 64)) == 656
    assert M.row_bytes(R(M.E4M3_S128, 128)) == 132
    assert M.row_bytes(R(M.E2M1_S16, 512)) == 288
    assert M.row_bytes(R(M.E2M1_S16, 128)) == 72
    assert M.row_bytes(R(M.MXFP4, 128)) == 68 and M.row_bytes(R(M.MXFP4, 48)) == -1
    assert M.row_bytes(R(M.MXFP8, 512)) == 528 and M.row_bytes(R(M.MXFP8, 40)) == -1
    assert M.row_bytes(R(M.BF16, 512, 64)) == 1152
    assert M.row_bytes(R(M.F32, 64, 16)) == 320
    assert M.row_bytes(R(M.E2M1_S16, 512, 64)) == -1          # no separate RoPE part in FP4 rows
    assert M.row_bytes(R(M.E4M3_S128, 100)) == -1
    assert M.row_bytes(R(7, 128)) == -1
    assert M.lib().mla_status_str(3) == b"workspace missing or too small"
    assert M.version() >= 100


def _row(M, fmt, dim, rope=0):
    return M._CRow(dim, rope, fmt)


def test_host_validation_rejects_before_launch(M):
    L = M.lib()
    fake = C.c_void_p(0x1000)                  # never dereferenced: validation fails first
    r_main, r_idx = _row(M, M.E4M3_S128, 512, 64), _row(M, M.E4M3_S128, 128)
    # append: negative batch
    assert L.mla_kv_append_quant(r_main, r_idx, fake, fake, fake, -1, 1, 10, fake, 6560, fake, 1320,
                                 None, None, None, 0, 0, 1, None) == 1
    # append: unsupported row format
    assert L.mla_kv_append_quant(_row(M, 9, 512), r_idx, fake, fake, fake, 1, 1, 10, fake, 6560, None, 0,
                                 None, None, None, 0, 0, 1, None) == 2
    # append: window without a ring
    assert L.mla_kv_append_quant(r_main, r_idx, None, None, None, 1, 0, 0, None, 0, None, 0,
                                 fake, fake, None, 128, 512, 1, None) == 1
    # append: window entries in a format other than BF16 / MXFP8, or an MXFP8 width not a multiple of 32
    assert L.mla_kv_append_quant(r_main, r_idx, None, None, None, 1, 0, 0, None, 0, None, 0,
                                 fake, fake, fake, 128, 512, 7, None) == 2
    assert L.mla_kv_append_quant(r_main, r_idx, None, None, None, 1, 0, 0, None, 0, None, 0,
                                 fake, fake, fake, 128, 520, M.MXFP8, None) == 2
    # decode: window entries in an unsupported format
    assert L.mla_sparse_decode(r_main, 512, C.c_void_p(0x10000), C.c_void_p(0x10000), 6560, 10, fake, 4,
                               fake, fake, 128, 7, 0.1, None, 1, 128, C.c_void_p(0x10000), fake,
                               C.c_void_p(0x100000), 1 << 30, None) == 2
    # decode: the MXFP8 window's bf16 copy is part of the workspace
    wb = L.mla_sparse_decode_workspace(r_main, 512, 4, 128, 2048, 128, M.BF16)
    w8 = L.mla_sparse_decode_workspace(r_main, 512, 4, 128, 2048, 128, M.MXFP8)
    assert w8 == wb + 4 * 128 * 576 * 2
    # compress: an empty window, negative eps, an odd rotation width, more than 2048 channels
    assert L.mla_compress_append(r_main, fake, fake, 0, None, 1e-6, 0, None, None, 1, 0, None, 0, fake, None) == 1
    assert L.mla_compress_append(r_main, fake, fake, 2, None, -1.0, 0, None, None, 1, 0, None, 0, fake, None) == 1
    assert L.mla_compress_append(r_main, fake, fake, 2, None, 1e-6, 3, fake, None, 1, 0, None, 0, fake, None) == 1
    assert L.mla_compress_append(_row(M, M.BF16, 4096), fake, fake, 2, None, 1e-6, 0, None, None, 1, 0, None, 0,
                                 fake, None) == 2
    assert L.mla_compress_append(_row(M, M.BF16, 2048), fake, fake, 2, None, 1e-6, 1024, fake, None, 1, 0, None, 0,
                                 fake, None) == 2
    # topk: score scale must be positive
    assert L.mla_indexer_topk(r_idx, fake, fake, 0.0, fake, 1408, 10, fake, None, 0, 1, 64, 8,
                              fake, None, fake, 1 << 20, None) == 1
    # topk: a pool size without a pool, and a negative pool size
    assert L.mla_indexer_topk(r_idx, fake, fake, 0.1, fake, 1408, 10, fake, None, 5, 1, 64, 8,
                              fake, None, fake, 1 << 20, None) == 1
    assert L.mla_indexer_topk(r_idx, fake, fake, 0.1, fake, 1408, 10, fake, fake, -1, 1, 64, 8,
                              fake, None, fake, 1 << 20, None) == 1
    # topk: a pool larger than the capacity sizes the workspace
    need = L.mla_indexer_topk_workspace(1, 100000, 8)
    assert need > L.mla_indexer_topk_workspace(1, 10, 8)
    assert L.mla_indexer_topk(r_idx, C.c_void_p(0x10000), fake, 0.1, C.c_void_p(0x10000), 1408, 10, fake,
                              fake, 100000, 1, 64, 8, fake, None, C.c_void_p(0x100000), need - 256, None) == 3
    # pool: block not a power of two, or over 64
    assert L.mla_indexer_pool(fake, 1000, fake, 1, 3, 16, fake, fake, 1 << 24, None) == 2
    assert L.mla_indexer_pool(fake, 1000, fake, 1, 128, 16, fake, fake, 1 << 24, None) == 2
    # pool: negative sizes, missing pointers, workspace too small
    assert L.mla_indexer_pool(fake, 1000, fake, 1, 8, -1, fake, fake, 1 << 24, None) == 1
    assert L.mla_indexer_pool(fake, -5, fake, 1, 8, 16, fake, fake, 1 << 24, None) == 1
    assert L.mla_indexer_pool(None, 1000, fake, 1, 8, 16, fake, fake, 1 << 24, None) == 1
    assert L.mla_indexer_pool(fake, 1000, fake, 1, 8, 16, fake, C.c_void_p(0x100000), 64, None) == 3
    # pool: nothing to select is a successful no-op (no launch)
    assert L.mla_indexer_pool(None, 1000, None, 1, 8, 0, None, None, 0, None) == 0
    assert L.mla_indexer_pool(None, 1000, None, 0, 8, 16, None, None, 0, None) == 0
    # topk: workspace too small
    assert L.mla_indexer_topk(r_idx, fake, fake, 0.1, C.c_void_p(0x10000), 1408, 10, fake, None, 0, 1, 64, 8,
                              fake, None, C.c_void_p(0x100000), 16, None) == 3
    assert b"workspace" in L.mla_last_error()
    # topk: no kernel for this shape (H_I * dim too large for the generic scan)
    assert L.mla_indexer_topk(_row(M, M.F32, 512), C.c_void_p(0x10000), fake, 0.1, C.c_void_p(0x10000),
                              20480, 10, fake, None, 0, 1, 64, 8, fake, None, C.c_void_p(0x100000),
                              1 << 24, None) == 2
    # append + topk: the indexer cache is required
    assert L.mla_append_indexer_topk(r_main, r_idx, fake, fake, fake, 1, fake, 6560, None, 0, 10,
                                     None, None, None, 0, 0, 1, fake, fake, 0.1, fake, 1, 64, 8,
                                     fake, None, fake, 1 << 20, None) == 1
    # append + topk: the append half is validated too (unsupported main row format)
    assert L.mla_append_indexer_topk(_row(M, 9, 512), r_idx, fake, fake, fake, 1, fake, 6560, fake, 1408, 10,
                                     None, None, None, 0, 0, 1, fake, fake, 0.1, fake, 1, 64, 8,
                                     fake, None, fake, 1 << 20, None) == 2
    # append + topk: and the top-k half (workspace too small)
    assert L.mla_append_indexer_topk(r_main, r_idx, fake, fake, fake, 1, C.c_void_p(0x10000), 6560,
                                     C.c_void_p(0x10000), 1408, 10, None, None, None, 0, 0, 1, fake, fake, 0.1,
                                     fake, 1, 64, 8, fake, None, C.c_void_p(0x100000), 16, None) == 3
    # decode: d_v larger than the latent
    assert L.mla_sparse_decode(r_main, 600, fake, fake, 6560, 10, fake, 4, None, None, 0, 1, 0.1, None, 1, 128,
                               fake, fake, fake, 1 << 30, None) == 1
    # decode: workspace too small for the MFMA path
    assert L.mla_sparse_decode(r_main, 512, C.c_void_p(0x10000), C.c_void_p(0x10000), 6560, 10, fake, 4,
                               None, None, 0, 1, 0.1, None, 1, 128, C.c_void_p(0x10000), fake,
                               C.c_void_p(0x100000), 64, None) == 3
    # decode: misaligned query
    assert L.mla_sparse_decode(r_main, 512, C.c_void_p(0x10002), C.c_void_p(0x10000), 6560, 10, fake, 4,
                               None, None, 0, 1, 0.1, None, 1, 128, C.c_void_p(0x10000), fake,
                               C.c_void_p(0x100000), 1 << 30, None) == 1
    # decode epilogue: misaligned sinks; output RoPE without its table, or of an unsupported width
    def epi(sinks, r, cs):
        e = M._CEpilogue(sinks, r, cs)
        return e, C.c_void_p(C.addressof(e))
    for (sk, r, cs), want in (((0x10002, 0, None), 1), ((None, 64, None), 1), ((None, -8, 0x20000), 1),
                              ((None, 12, 0x20000), 2), ((None, 512, 0x20000), 2)):
        keep, ep = epi(sk, r, cs)
        assert L.mla_sparse_decode(r_main, 512, C.c_void_p(0x10000), C.c_void_p(0x10000), 6560, 10, fake, 4,
                                   None, None, 0, 1, 0.1, ep, 1, 128, C.c_void_p(0x10000), fake,
                                   C.c_void_p(0x100000), 1 << 30, None) == want, (sk, r, cs)


def test_group_step_rejects_before_launch(M):
    """mla_csa2_group_step checks the group and every layer before its first launch."""
    L = M.lib()
    r_main, r_idx = _row(M, M.E2M1_S16, 512), _row(M, M.E2M1_S16, 128)
    a, fake = 0x10000, C.c_void_p(0x10000)

    def layer(mode, q=a, win=None):
        return M._CLayer(mode, q, a, a, a, a, win, a if win else None)

    def call(layers, W=0, topk_bytes=1 << 30, dec_bytes=1 << 30, idx_b=fake, pool=(0, 8, None, None)):
        arr = (M._CLayer * len(layers))(*layers)
        return L.mla_csa2_group_step(r_main, r_idx, 512, len(layers), C.cast(arr, C.c_void_p), fake, fake, fake, 1,
                                     fake, 288 * 1000, fake, 72 * 1000, 1000, fake, 2, 64, 64, 512, 0.1, 0.04,
                                     fake, fake, W, M.BF16, 0, *pool, fake, idx_b, C.c_void_p(0x100000), topk_bytes,
                                     C.c_void_p(0x200000), dec_bytes, None)
    full, reuse = 0, 2
    assert call([layer(full), layer(7)]) == 1                       # unknown mode
    assert b"mode" in L.mla_last_error()
    assert call([layer(reuse), layer(full)]) == 1                   # nothing selected yet
    assert call([layer(full), layer(reuse, q=a + 2)]) == 1          # misaligned query
    assert call([layer(full), layer(reuse)], W=128) == 1            # a window without rings
    assert call([layer(full)], idx_b=None) == 1                     # one index buffer
    assert call([layer(full)], pool=(16, 8, None, None)) == 1       # a pool without its arrays
    assert call([], W=0) == 1                                       # no layers
    assert call([layer(full), layer(reuse)], topk_bytes=64) == 3    # short workspaces
    assert call([layer(full), layer(reuse)], dec_bytes=64) == 3
    assert b"decode workspace" in L.mla_last_error()


def test_workspace_queries(M):
    assert M.mla_indexer_topk_workspace(4, 131072, 2048) >= 4 * 131072 * (4 + 8)
    # the pool's selection runs over capacity / block block scores
    assert M.mla_indexer_pool_workspace(1, 524288, 8) >= M.mla_indexer_topk_workspace(1, 65536, 2048)
    assert M.mla_indexer_pool_workspace(1, 524288, 8) < M.mla_indexer_topk_workspace(1, 524288, 2048)
    r = M.Row(M.E4M3_S128, 512, 64)
    assert M.mla_sparse_decode_workspace(r, 512, 4, 128, 2048, 0) >= 4 * 128 * 512 * 4
    assert M.mla_sparse_decode_workspace(M.Row(M.F32, 64, 16), 64, 1, 16, 32, 0) == 0   # generic path


def test_profile_hooks_off_by_default_and_reject_unknown_names(M):
    # nothing has been launched in this process, so every count is zero and no
    # event is ever waited on
    M.mla_profile_enable(())
    for name in M.PROFILE_KERNELS:
        assert M.mla_profile_read(name) == (0, 0.0)
    # the header's mask bits follow the binding's names
    text = open(HEADER).read()
    for bit, name in enumerate(M.PROFILE_KERNELS):
        assert re.search(rf"#define MLA_PROF_{name.upper()} 0x{1 << bit:02x}\b", text), name
    with pytest.raises(M.MLAError, match="unknown kernel name"):
        M.mla_profile_read("k_scan")
    n, ms = C.c_int32(), C.c_double()
    assert M.lib().mla_profile_read(None, C.byref(n), C.byref(ms)) == 1


def test_options_set_get_and_validation(M):
    """Kernel-choice options: declared names round-trip, unknown names and values
    out of range are rejected on the host, and 0 restores the default."""
    for name, v in (("topk_path", 2), ("topk_final", 1), ("scan_queues", 1), ("scan_blocks", 300),
                    ("decode_rows_per_split", 128)):
        assert M.mla_get_option(name) == 0
        with M.option(name, v):
            assert M.mla_get_option(name) == v
        assert M.mla_get_option(name) == 0
    with pytest.raises(M.MLAError, match="unknown option"):
        M.mla_set_option("no_such_option", 1)
    with pytest.raises(M.MLAError, match="out of range"):
        M.mla_set_option("topk_path", 3)
    with pytest.raises(M.MLAError, match="out of range"):
        M.mla_set_option("scan_blocks", -1)
    assert M.mla_last_kernels() == []                          # nothing launched on this thread
