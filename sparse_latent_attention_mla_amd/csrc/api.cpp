// api.cpp -- the C ABI of include/mla.h: argument validation on the host,
// workspace carving, dispatch to the gfx950 launchers, error reporting.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "launch.hpp"
#include "mla.h"

namespace {

thread_local char g_err[512] = "";

mla_status_t fail(mla_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

mla_status_t ok() {
    g_err[0] = '\0';
    return MLA_OK;
}

mla_status_t hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return ok();
    return fail(MLA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Alignment every row start keeps when the cache base is 16-byte aligned and
// the sequence stride is a multiple of it: the largest power of two <= 16
// dividing the row size.  The kernels never load wider than this from a row.
int64_t row_alignment(int64_t row_bytes) {
    int64_t a = 16;
    while (a > 1 && row_bytes % a != 0) a >>= 1;
    return a;
}

// shared: a stride of 0 is accepted (every batch row reads the same sequence's
// rows: several queries of one sequence); only for calls that do not write rows.
mla_status_t check_rows(const char* what, mla_row_t row, const void* cache, int64_t stride, int64_t capacity,
                        int B, int64_t* row_bytes, bool shared = false) {
    const int64_t rb = mla_row_bytes(row);
    if (rb < 0)
        return fail(MLA_ERR_UNSUPPORTED, "%s: unsupported row format (fmt %d, dim %d, rope %d)", what, row.fmt,
                    row.dim, row.rope_dim);
    *row_bytes = rb;
    if (!cache) return ok();
    if (capacity < 0) return fail(MLA_ERR_INVALID_ARG, "%s: capacity < 0", what);
    if (B > 1 && stride < capacity * rb && !(shared && stride == 0))
        return fail(MLA_ERR_INVALID_ARG, "%s: sequence stride %lld < capacity * row bytes %lld", what,
                    (long long)stride, (long long)(capacity * rb));
    const int64_t ra = row_alignment(rb);
    if (!aligned(cache, 16) || stride % ra != 0)
        return fail(MLA_ERR_INVALID_ARG, "%s: cache base must be 16-byte aligned and the sequence stride a "
                    "multiple of %lld", what, (long long)ra);
    return ok();
}

struct TopkLayout {
    size_t queues, scores, hist, counts, sel, cand, cand2, total;
};

TopkLayout topk_layout(int32_t B, int64_t capacity) {
    TopkLayout L;
    const size_t b = B > 0 ? (size_t)B : 0, cap = capacity > 0 ? (size_t)capacity : 0;
    const size_t groups = capacity > 0 ? (size_t)mla::select_groups(capacity) : 0;
    // the scan's work queues and the histogram first, at places that depend on
    // nothing but the sequence, so that what a call leaves zeroed stays the
    // queues and the histogram whatever the next call's sizes
    L.queues = 0;
    L.hist = L.queues + (size_t)mla::kScanQueuesHost * mla::kQueueWordsHost * sizeof(uint32_t);
    L.scores = L.hist + round256(b * (size_t)mla::kHistWordsHost * sizeof(uint32_t));
    L.counts = L.scores + round256(b * cap * sizeof(float));
    L.sel = L.counts + round256(b * groups * 2 * sizeof(uint32_t));
    L.cand = L.sel + round256(b * cap * sizeof(int32_t));
    L.cand2 = L.cand + round256(b * cap * sizeof(uint64_t));
    L.total = L.cand2 + round256(b * cap * sizeof(uint64_t));
    return L;
}

// Validated argument block of the quantise-append.
mla_status_t append_args(mla_row_t main_row, mla_row_t idx_row, const float* new_main, const float* new_idx,
                         const int32_t* slots, int32_t B, int32_t n_new, int64_t capacity, void* main_cache,
                         int64_t main_seq_stride, void* idx_cache, int64_t idx_seq_stride, const float* new_win,
                         const int32_t* win_pos, void* win_ring, int32_t W, int32_t Dw, int32_t win_fmt,
                         mla::AppendArgs* out) {
    if (B < 0 || n_new < 0) return fail(MLA_ERR_INVALID_ARG, "append: B and n_new must be >= 0");
    mla::AppendArgs a{};
    if (main_cache) {
        mla_status_t s = check_rows("append main", main_row, main_cache, main_seq_stride, capacity, B,
                                    &a.main_row_bytes);
        if (s != MLA_OK) return s;
        if (main_row.dim + main_row.rope_dim > 4096)
            return fail(MLA_ERR_UNSUPPORTED, "append: main row wider than 4096 channels");
        if (!new_main) return fail(MLA_ERR_INVALID_ARG, "append: new_main is NULL");
    }
    if (idx_cache) {
        if (idx_row.rope_dim != 0) return fail(MLA_ERR_INVALID_ARG, "append: indexer rows have no RoPE part");
        mla_status_t s = check_rows("append indexer", idx_row, idx_cache, idx_seq_stride, capacity, B,
                                    &a.idx_row_bytes);
        if (s != MLA_OK) return s;
        if (!new_idx) return fail(MLA_ERR_INVALID_ARG, "append: new_idx is NULL");
    }
    if ((main_cache || idx_cache) && n_new > 0 && B > 0 && !slots)
        return fail(MLA_ERR_INVALID_ARG, "append: slots is NULL");
    if (new_win) {
        if (!win_pos || !win_ring) return fail(MLA_ERR_INVALID_ARG, "append: window needs win_pos and win_ring");
        if (W <= 0 || Dw <= 0) return fail(MLA_ERR_INVALID_ARG, "append: window needs W > 0 and Dw > 0");
        if (win_fmt != MLA_FMT_BF16 && win_fmt != MLA_FMT_MXFP8)
            return fail(MLA_ERR_UNSUPPORTED, "append: window entries must be BF16 or MXFP8");
        if (win_fmt == MLA_FMT_MXFP8 && (Dw % 32 != 0 || Dw > 2048))
            return fail(MLA_ERR_UNSUPPORTED, "append: an MXFP8 window needs Dw % 32 == 0 and Dw <= 2048");
        if (win_fmt == MLA_FMT_BF16 && !aligned(win_ring, 2))
            return fail(MLA_ERR_INVALID_ARG, "append: misaligned window ring");
    }
    a.main_fmt = main_row.fmt;
    a.main_dim = main_row.dim;
    a.main_rope = main_row.rope_dim;
    a.idx_fmt = idx_row.fmt;
    a.idx_dim = idx_row.dim;
    a.new_main = new_main;
    a.new_idx = new_idx;
    a.slots = slots;
    a.B = B;
    a.n_new = n_new;
    a.capacity = capacity;
    a.main_cache = static_cast<uint8_t*>(main_cache);
    a.main_stride = main_seq_stride;
    a.idx_cache = static_cast<uint8_t*>(idx_cache);
    a.idx_stride = idx_seq_stride;
    a.new_win = new_win;
    a.win_pos = win_pos;
    a.win_ring = new_win ? static_cast<uint16_t*>(win_ring) : nullptr;
    a.W = W;
    a.Dw = Dw;
    a.win_fmt = win_fmt;
    *out = a;
    return ok();
}

// Validated scan and selection of one top-k call (empty: nothing to compute).
struct TopkCall {
    bool empty = false;
    mla::ScanArgs scan{};
    mla::TopkWorkspace ws{};
    int32_t* out_idx = nullptr;
};

mla_status_t topk_args(mla_row_t idx_row, const void* q_idx, const float* w, float score_scale,
                       const void* idx_cache, int64_t idx_seq_stride, int64_t capacity, const int32_t* n_visible,
                       const int32_t* cand, int32_t n_cand, int32_t B, int32_t H_I, int32_t k, int32_t* out_idx,
                       float* out_scores, void* workspace, size_t workspace_bytes, TopkCall* out,
                       bool score_bf16 = false) {
    if (B < 0 || k < 0 || H_I < 1 || capacity < 0)
        return fail(MLA_ERR_INVALID_ARG, "indexer_topk: need B >= 0, k >= 0, H_I >= 1, capacity >= 0");
    if (n_cand < 0 || (!cand && n_cand != 0))
        return fail(MLA_ERR_INVALID_ARG, "indexer_topk: a candidate pool needs cand != NULL and n_cand >= 0");
    if (!(score_scale > 0.0f)) return fail(MLA_ERR_INVALID_ARG, "indexer_topk: score_scale must be > 0");
    if (idx_row.rope_dim != 0) return fail(MLA_ERR_INVALID_ARG, "indexer_topk: indexer rows have no RoPE part");
    if (B == 0 || k == 0) {
        out->empty = true;
        return ok();
    }
    int64_t rb = 0;
    mla_status_t s = check_rows("indexer_topk", idx_row, idx_cache, idx_seq_stride, capacity, B, &rb, true);
    if (s != MLA_OK) return s;
    if (!q_idx || !w || !idx_cache || !n_visible || !out_idx)
        return fail(MLA_ERR_INVALID_ARG, "indexer_topk: a required pointer is NULL");
    if (!aligned(q_idx, 16)) return fail(MLA_ERR_INVALID_ARG, "indexer_topk: q_idx must be 16-byte aligned");
    if (!mla::scan_supported(idx_row.fmt, idx_row.dim, H_I))
        return fail(MLA_ERR_UNSUPPORTED, "indexer_topk: no kernel for fmt %d, dim %d, H_I %d", idx_row.fmt,
                    idx_row.dim, H_I);
    if (capacity > (int64_t)0x7FFFFFFF) return fail(MLA_ERR_UNSUPPORTED, "indexer_topk: capacity over 2^31-1");
    // with a pool the scores and the selection's lists have n_cand entries per sequence
    const int64_t rows = cand ? std::max<int64_t>(capacity, n_cand) : capacity;
    const TopkLayout L = topk_layout(B, rows);
    if (!workspace || workspace_bytes < L.total || !aligned(workspace, 256))
        return fail(MLA_ERR_WORKSPACE, "indexer_topk: workspace needs %zu bytes, 256-byte aligned", L.total);
    if (out_scores && !aligned(out_scores, 4)) return fail(MLA_ERR_INVALID_ARG, "indexer_topk: misaligned out_scores");
    char* ws = static_cast<char*>(workspace);
    mla::TopkWorkspace& T = out->ws;
    T.scores = out_scores ? out_scores : reinterpret_cast<float*>(ws + L.scores);
    T.hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    T.counts = reinterpret_cast<uint32_t*>(ws + L.counts);
    T.sel = reinterpret_cast<int32_t*>(ws + L.sel);
    T.cand = reinterpret_cast<uint64_t*>(ws + L.cand);
    T.cand2 = reinterpret_cast<uint64_t*>(ws + L.cand2);
    mla::ScanArgs& a = out->scan;
    a.fmt = idx_row.fmt;
    a.dim = idx_row.dim;
    a.row_bytes = rb;
    a.q_idx = q_idx;
    a.w = w;
    a.sigma = score_scale;
    a.cache = static_cast<const uint8_t*>(idx_cache);
    a.stride = idx_seq_stride;
    a.capacity = capacity;
    a.n_visible = n_visible;
    a.B = B;
    a.H_I = H_I;
    a.k = k;
    a.scores = T.scores;
    a.hist = T.hist;
    a.queues = reinterpret_cast<uint32_t*>(ws + L.queues);
    a.cand = cand;
    a.n_cand = cand ? n_cand : 0;
    a.score_bf16 = score_bf16 ? 1 : 0;
    out->out_idx = out_idx;
    return ok();
}

// A selection whose final is left to the decode that follows (groups > 0: k_select ran
// alone, its lists and counts in ws).
struct Deferred {
    int groups = 0;
    mla::TopkWorkspace ws{};
    const int32_t* n_visible = nullptr;
    int64_t capacity = 0;
};

// The scan (carrying `append` when given) and the selection; with `defer`, only
// k_select when the selection takes its many-workgroup path over every entry.
mla_status_t topk_launch(const TopkCall& c, const mla::AppendArgs* append, hipStream_t st,
                         Deferred* defer = nullptr) {
    hipError_t e = mla::launch_scan(c.scan, st, append);
    if (e != hipSuccess) return hip_status(e, "indexer scan");
    const mla::ScanArgs& a = c.scan;
    if (defer && !a.cand) {
        defer->groups = 0;
        e = mla::launch_select_lists(a.scores, a.capacity, a.n_visible, a.B, a.k, c.ws, st, &defer->groups);
        if (e != hipSuccess) return hip_status(e, "top-k select");
        if (defer->groups > 0) {
            defer->ws = c.ws;
            defer->n_visible = a.n_visible;
            defer->capacity = a.capacity;
            return ok();
        }
    }
    if (a.cand) {       // the pool's n_cand entries, reported as their positions
        mla::SelectMap map;
        map.cand = a.cand;
        map.n_visible = a.n_visible;
        map.limit = a.capacity;
        e = mla::launch_select(a.scores, a.n_cand, nullptr, a.B, a.k, c.ws, c.out_idx, st, map);
    } else {
        e = mla::launch_select(a.scores, a.capacity, a.n_visible, a.B, a.k, c.ws, c.out_idx, st);
    }
    return hip_status(e, "top-k select");
}

// Scratch of mla_sparse_decode_noalloc: one array per GPU, kept until the
// process ends. Host code never passes the array's name to a kernel (on the
// host it only stands in for the symbol); the device address of each GPU's copy
// is looked up once, with that GPU current, and kept.
constexpr size_t kScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The calling thread's current device's scratch address, or null (error set).
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        fail(MLA_ERR_HIP, "sparse_decode_noalloc: no current device (or device index >= %d)", kMaxDevices);
        return nullptr;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            fail(MLA_ERR_HIP, "sparse_decode_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace

extern "C" {

int64_t mla_row_bytes(mla_row_t row) {
    if (row.dim <= 0 || row.rope_dim < 0 || row.dim > 8192 || row.rope_dim > 8192) return -1;
    switch (row.fmt) {
    case MLA_FMT_F32: return 4LL * (row.dim + row.rope_dim);
    case MLA_FMT_BF16: return 2LL * (row.dim + row.rope_dim);
    case MLA_FMT_E4M3_S128:
        if (row.dim % 128 != 0 || row.rope_dim % 2 != 0) return -1;
        return (int64_t)row.dim + 4LL * (row.dim / 128) + 2LL * row.rope_dim;
    case MLA_FMT_E2M1_S16:
        if (row.dim % 16 != 0 || row.rope_dim != 0 || row.dim > 1024) return -1;
        return (int64_t)row.dim / 2 + row.dim / 16;
    case MLA_FMT_MXFP4:
        if (row.dim % 32 != 0 || row.rope_dim != 0 || row.dim > 1024) return -1;
        return (int64_t)row.dim / 2 + row.dim / 32;
    case MLA_FMT_MXFP8:
        if (row.dim % 32 != 0 || row.rope_dim != 0 || row.dim > 2048) return -1;
        return (int64_t)row.dim + row.dim / 32;
    default: return -1;
    }
}

const char* mla_status_str(int32_t status) {
    switch (status) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported format or shape";
    case MLA_ERR_WORKSPACE: return "workspace missing or too small";
    case MLA_ERR_HIP: return "HIP error";
    default: return "unknown status";
    }
}

const char* mla_last_error(void) { return g_err; }

mla_status_t mla_profile_enable(int32_t kernels) {
    mla::prof_enable(static_cast<uint32_t>(kernels));
    return ok();
}

mla_status_t mla_profile_read(const char* kernel, int32_t* launches, double* total_ms) {
    if (!kernel || !launches || !total_ms) return fail(MLA_ERR_INVALID_ARG, "mla_profile_read: NULL argument");
    const int k = mla::prof_index(kernel);
    if (k < 0) return fail(MLA_ERR_INVALID_ARG, "mla_profile_read: unknown kernel name '%s'", kernel);
    return hip_status(mla::prof_read(k, launches, total_ms), "mla_profile_read");
}

int32_t mla_version(void) { return 105; }

mla_status_t mla_set_option(const char* name, int64_t value) {
    if (!name) return fail(MLA_ERR_INVALID_ARG, "mla_set_option: NULL name");
    const int i = mla::option_index(name);
    if (i < 0) return fail(MLA_ERR_INVALID_ARG, "mla_set_option: unknown option '%s'", name);
    if (!mla::option_set(i, value))
        return fail(MLA_ERR_INVALID_ARG, "mla_set_option: value %lld out of range for '%s'", (long long)value, name);
    return ok();
}

mla_status_t mla_get_option(const char* name, int64_t* value) {
    if (!name || !value) return fail(MLA_ERR_INVALID_ARG, "mla_get_option: NULL argument");
    const int i = mla::option_index(name);
    if (i < 0) return fail(MLA_ERR_INVALID_ARG, "mla_get_option: unknown option '%s'", name);
    *value = mla::option(static_cast<mla::Opt>(i));
    return ok();
}

const char* mla_last_kernels(void) { return mla::launched_names(); }

mla_status_t mla_kv_append_quant(mla_row_t main_row, mla_row_t idx_row, const float* new_main,
                                 const float* new_idx, const int32_t* slots, int32_t B, int32_t n_new,
                                 int64_t capacity, void* main_cache, int64_t main_seq_stride, void* idx_cache,
                                 int64_t idx_seq_stride, const float* new_win, const int32_t* win_pos,
                                 void* win_ring, int32_t W, int32_t Dw, int32_t win_fmt, void* stream) {
    mla::begin_call();
    mla::AppendArgs a{};
    const mla_status_t s = append_args(main_row, idx_row, new_main, new_idx, slots, B, n_new, capacity, main_cache,
                                       main_seq_stride, idx_cache, idx_seq_stride, new_win, win_pos, win_ring, W,
                                       Dw, win_fmt, &a);
    if (s != MLA_OK) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    return hip_status(mla::launch_append(a, st), "append launch");
}

mla_status_t mla_compress_append(mla_row_t main_row, const float* kv, const float* gate, int32_t m,
                                 const float* norm_weight, float eps, int32_t rope_dim, const float* rope_cs,
                                 const int32_t* slots, int32_t B, int64_t capacity, void* main_cache,
                                 int64_t main_seq_stride, float* out_entry, void* stream) {
    mla::begin_call();
    if (B < 0 || m < 1 || !(eps >= 0.0f) || capacity < 0)
        return fail(MLA_ERR_INVALID_ARG, "compress: need B >= 0, m >= 1, eps >= 0, capacity >= 0");
    const int64_t rb = mla_row_bytes(main_row);
    if (rb < 0 || main_row.fmt == MLA_FMT_MXFP8) return fail(MLA_ERR_UNSUPPORTED, "compress: unsupported row format");
    const int D = main_row.dim + main_row.rope_dim;
    if (D > 2048) return fail(MLA_ERR_UNSUPPORTED, "compress: more than 2048 channels");
    if (rope_dim < 0 || rope_dim % 2 != 0 || rope_dim > D || (rope_dim > 0 && !rope_cs))
        return fail(MLA_ERR_INVALID_ARG, "compress: rope_dim must be even, <= D, with rope_cs");
    if (rope_dim > 512) return fail(MLA_ERR_UNSUPPORTED, "compress: rope_dim above 512");
    if (B == 0) return ok();
    if (!kv || !gate) return fail(MLA_ERR_INVALID_ARG, "compress: kv and gate are required");
    if (main_cache) {
        int64_t rb2 = 0;
        const mla_status_t s = check_rows("compress", main_row, main_cache, main_seq_stride, capacity, B, &rb2);
        if (s != MLA_OK) return s;
        if (!slots) return fail(MLA_ERR_INVALID_ARG, "compress: slots is NULL");
    }
    mla::CompressArgs a{};
    a.fmt = main_row.fmt;
    a.dim = main_row.dim;
    a.rope = main_row.rope_dim;
    a.row_bytes = rb;
    a.kv = kv;
    a.gate = gate;
    a.g = norm_weight;
    a.eps = eps;
    a.m = m;
    a.D = D;
    a.rope_dim = rope_dim;
    a.rope_cs = rope_cs;
    a.slots = main_cache ? slots : nullptr;
    a.capacity = capacity;
    a.cache = static_cast<uint8_t*>(main_cache);
    a.stride = main_seq_stride;
    a.out = out_entry;
    a.B = B;
    return hip_status(mla::launch_compress(a, static_cast<hipStream_t>(stream)), "compress launch");
}

size_t mla_indexer_topk_workspace(int32_t B, int64_t capacity, int32_t k) {
    (void)k;
    return topk_layout(B, capacity).total;
}

static mla_status_t indexer_topk(mla_row_t idx_row, const void* q_idx, const float* w, float score_scale,
                                 const void* idx_cache, int64_t idx_seq_stride, int64_t capacity,
                                 const int32_t* n_visible, const int32_t* cand, int32_t n_cand, int32_t B,
                                 int32_t H_I, int32_t k, int32_t* out_idx, float* out_scores, void* workspace,
                                 size_t workspace_bytes, void* stream, bool score_bf16, Deferred* defer = nullptr) {
    mla::begin_call();
    TopkCall c;
    const mla_status_t s = topk_args(idx_row, q_idx, w, score_scale, idx_cache, idx_seq_stride, capacity, n_visible,
                                     cand, n_cand, B, H_I, k, out_idx, out_scores, workspace, workspace_bytes, &c,
                                     score_bf16);
    if (s != MLA_OK || c.empty) return s;
    return topk_launch(c, nullptr, static_cast<hipStream_t>(stream), defer);
}

mla_status_t mla_indexer_topk(mla_row_t idx_row, const void* q_idx, const float* w, float score_scale,
                              const void* idx_cache, int64_t idx_seq_stride, int64_t capacity,
                              const int32_t* n_visible, const int32_t* cand, int32_t n_cand, int32_t B,
                              int32_t H_I, int32_t k, int32_t* out_idx, float* out_scores, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return indexer_topk(idx_row, q_idx, w, score_scale, idx_cache, idx_seq_stride, capacity, n_visible, cand, n_cand,
                        B, H_I, k, out_idx, out_scores, workspace, workspace_bytes, stream, false);
}

mla_status_t mla_indexer_topk_bf16(mla_row_t idx_row, const void* q_idx, const float* w, float score_scale,
                                   const void* idx_cache, int64_t idx_seq_stride, int64_t capacity,
                                   const int32_t* n_visible, const int32_t* cand, int32_t n_cand, int32_t B,
                                   int32_t H_I, int32_t k, int32_t* out_idx, float* out_scores, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    return indexer_topk(idx_row, q_idx, w, score_scale, idx_cache, idx_seq_stride, capacity, n_visible, cand, n_cand,
                        B, H_I, k, out_idx, out_scores, workspace, workspace_bytes, stream, true);
}

static mla_status_t append_indexer_topk(mla_row_t main_row, mla_row_t idx_row, const float* new_main,
                                        const float* new_idx, const int32_t* slots, int32_t n_new, void* main_cache,
                                        int64_t main_seq_stride, void* idx_cache, int64_t idx_seq_stride,
                                        int64_t capacity, const float* new_win, const int32_t* win_pos,
                                        void* win_ring, int32_t W, int32_t Dw, int32_t win_fmt, const void* q_idx,
                                        const float* w, float score_scale, const int32_t* n_visible, int32_t B,
                                        int32_t H_I, int32_t k, int32_t* out_idx, float* out_scores,
                                        void* workspace, size_t workspace_bytes, void* stream, bool score_bf16,
                                        Deferred* defer = nullptr) {
    mla::begin_call();
    if (!idx_cache) return fail(MLA_ERR_INVALID_ARG, "append_indexer_topk: idx_cache is NULL");
    mla::AppendArgs ap{};
    mla_status_t s = append_args(main_row, idx_row, new_main, new_idx, slots, B, n_new, capacity, main_cache,
                                 main_seq_stride, idx_cache, idx_seq_stride, new_win, win_pos, win_ring, W, Dw,
                                 win_fmt, &ap);
    if (s != MLA_OK) return s;
    TopkCall c;
    s = topk_args(idx_row, q_idx, w, score_scale, idx_cache, idx_seq_stride, capacity, n_visible, nullptr, 0, B,
                  H_I, k, out_idx, out_scores, workspace, workspace_bytes, &c, score_bf16);
    if (s != MLA_OK) return s;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (c.empty) return hip_status(mla::launch_append(ap, st), "append launch");
    if (n_new == 0) {                                      // at most a window entry: nothing to carry
        const mla_status_t sa = hip_status(mla::launch_append(ap, st), "append launch");
        if (sa != MLA_OK) return sa;
        return topk_launch(c, nullptr, st, defer);
    }
    return topk_launch(c, &ap, st, defer);
}

mla_status_t mla_append_indexer_topk(mla_row_t main_row, mla_row_t idx_row, const float* new_main,
                                     const float* new_idx, const int32_t* slots, int32_t n_new, void* main_cache,
                                     int64_t main_seq_stride, void* idx_cache, int64_t idx_seq_stride,
                                     int64_t capacity, const float* new_win, const int32_t* win_pos,
                                     void* win_ring, int32_t W, int32_t Dw, int32_t win_fmt, const void* q_idx,
                                     const float* w,
                                     float score_scale, const int32_t* n_visible, int32_t B, int32_t H_I,
                                     int32_t k, int32_t* out_idx, float* out_scores, void* workspace,
                                     size_t workspace_bytes, void* stream) {
    return append_indexer_topk(main_row, idx_row, new_main, new_idx, slots, n_new, main_cache, main_seq_stride,
                               idx_cache, idx_seq_stride, capacity, new_win, win_pos, win_ring, W, Dw, win_fmt, q_idx,
                               w, score_scale, n_visible, B, H_I, k, out_idx, out_scores, workspace, workspace_bytes,
                               stream, false);
}

mla_status_t mla_append_indexer_topk_bf16(mla_row_t main_row, mla_row_t idx_row, const float* new_main,
                                          const float* new_idx, const int32_t* slots, int32_t n_new,
                                          void* main_cache, int64_t main_seq_stride, void* idx_cache,
                                          int64_t idx_seq_stride, int64_t capacity, const float* new_win,
                                          const int32_t* win_pos, void* win_ring, int32_t W, int32_t Dw,
                                          int32_t win_fmt, const void* q_idx, const float* w, float score_scale,
                                          const int32_t* n_visible, int32_t B, int32_t H_I, int32_t k,
                                          int32_t* out_idx, float* out_scores, void* workspace,
                                          size_t workspace_bytes, void* stream) {
    return append_indexer_topk(main_row, idx_row, new_main, new_idx, slots, n_new, main_cache, main_seq_stride,
                               idx_cache, idx_seq_stride, capacity, new_win, win_pos, win_ring, W, Dw, win_fmt, q_idx,
                               w, score_scale, n_visible, B, H_I, k, out_idx, out_scores, workspace, workspace_bytes,
                               stream, true);
}

size_t mla_indexer_pool_workspace(int32_t B, int64_t capacity, int32_t block) {
    if (B < 0 || capacity < 0 || block < 1) return 0;
    const int64_t nb = (capacity + block - 1) / block;
    return topk_layout(B, nb).total + round256((size_t)B * sizeof(int32_t));
}

mla_status_t mla_indexer_pool(const float* scores, int64_t capacity, const int32_t* n_visible, int32_t B,
                              int32_t block, int32_t n_blocks, int32_t* out_pos, void* workspace,
                              size_t workspace_bytes, void* stream) {
    mla::begin_call();
    if (B < 0 || capacity < 0 || n_blocks < 0)
        return fail(MLA_ERR_INVALID_ARG, "indexer_pool: need B >= 0, capacity >= 0, n_blocks >= 0");
    if (block < 1 || block > 64 || (block & (block - 1)) != 0)
        return fail(MLA_ERR_UNSUPPORTED, "indexer_pool: block must be a power of two <= 64");
    if (capacity > (int64_t)0x7FFFFFFF || (int64_t)n_blocks * block > (int64_t)0x7FFFFFFF)
        return fail(MLA_ERR_UNSUPPORTED, "indexer_pool: capacity and n_blocks * block must be below 2^31");
    if (B == 0 || n_blocks == 0) return ok();
    if (!scores || !n_visible || !out_pos) return fail(MLA_ERR_INVALID_ARG, "indexer_pool: a required pointer is NULL");
    if (!aligned(scores, 4) || !aligned(out_pos, 4))
        return fail(MLA_ERR_INVALID_ARG, "indexer_pool: misaligned scores or out_pos");
    const int64_t nb = (capacity + block - 1) / block;
    const TopkLayout L = topk_layout(B, nb);
    const size_t need = mla_indexer_pool_workspace(B, capacity, block);
    if (!workspace || workspace_bytes < need || !aligned(workspace, 256))
        return fail(MLA_ERR_WORKSPACE, "indexer_pool: workspace needs %zu bytes, 256-byte aligned", need);
    char* ws = static_cast<char*>(workspace);
    mla::TopkWorkspace T;
    T.scores = reinterpret_cast<float*>(ws + L.scores);          // the block scores
    T.hist = reinterpret_cast<uint32_t*>(ws + L.hist);
    T.counts = reinterpret_cast<uint32_t*>(ws + L.counts);
    T.sel = reinterpret_cast<int32_t*>(ws + L.sel);
    T.cand = reinterpret_cast<uint64_t*>(ws + L.cand);
    T.cand2 = reinterpret_cast<uint64_t*>(ws + L.cand2);
    int32_t* nvb = reinterpret_cast<int32_t*>(ws + L.total);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = mla::launch_block_max(scores, capacity, n_visible, B, block, T.scores, nvb, T.hist, st);
    if (e != hipSuccess) return hip_status(e, "pool block maxima");
    mla::SelectMap map;
    map.expand = block;
    e = mla::launch_select(T.scores, nb, nvb, B, n_blocks, T, out_pos, st, map);
    return hip_status(e, "pool select");
}

// Bytes of the bf16 copy of an MXFP8 window ring, placed after the decode's own workspace.
static size_t window_copy_bytes(int32_t win_fmt, int32_t B, int32_t W, int D) {
    if (win_fmt != MLA_FMT_MXFP8 || W <= 0) return 0;
    return ((size_t)B * W * D * 2 + 255) & ~(size_t)255;
}

size_t mla_sparse_decode_workspace(mla_row_t main_row, int32_t d_v, int32_t B, int32_t H, int32_t k, int32_t W,
                                   int32_t win_fmt) {
    if (B <= 0 || H <= 0 || k < 0 || W < 0 || mla_row_bytes(main_row) < 0) return 0;
    return mla::decode_workspace_bytes(main_row.fmt, main_row.dim, main_row.rope_dim, d_v, B, H, k, W) +
           window_copy_bytes(win_fmt, B, W, main_row.dim + main_row.rope_dim);
}

static mla_status_t decode_impl(mla_row_t main_row, int32_t d_v, const void* q, const void* main_cache,
                                int64_t main_seq_stride, int64_t capacity, const int32_t* idx, int32_t k,
                                const float* new_win, const int32_t* win_pos, const void* win_ring,
                                const int32_t* win_len, int32_t W, int32_t win_fmt, float softmax_scale,
                                const mla_decode_epilogue_t* epilogue, int32_t B, int32_t H, float* out, float* lse,
                                void* workspace, size_t workspace_bytes, void* stream,
                                const Deferred* sel = nullptr, int32_t* idx_out = nullptr) {
    if (B < 0 || H < 1 || k < 0 || capacity < 0)
        return fail(MLA_ERR_INVALID_ARG, "sparse_decode: need B >= 0, H >= 1, k >= 0, capacity >= 0");
    const int D = main_row.dim + main_row.rope_dim;
    if (d_v <= 0 || d_v > main_row.dim) return fail(MLA_ERR_INVALID_ARG, "sparse_decode: need 0 < d_v <= dim");
    int64_t rb = 0;
    mla_status_t s = check_rows("sparse_decode", main_row, main_cache, main_seq_stride, capacity, B, &rb, true);
    if (s != MLA_OK) return s;
    if (B == 0) return ok();
    const bool finish = sel && sel->groups > 0;            // the rows come from the selection's lists
    if (!q || !out || !lse || (k > 0 && ((!idx && !finish) || !main_cache)) || (finish && !idx_out))
        return fail(MLA_ERR_INVALID_ARG, "sparse_decode: a required pointer is NULL");
    if (win_ring && (!win_len || W <= 0))
        return fail(MLA_ERR_INVALID_ARG, "sparse_decode: window needs win_len and W > 0");
    if (win_ring && win_fmt != MLA_FMT_BF16 && win_fmt != MLA_FMT_MXFP8)
        return fail(MLA_ERR_UNSUPPORTED, "sparse_decode: window entries must be BF16 or MXFP8");
    if (win_ring && win_fmt == MLA_FMT_MXFP8 && D % 32 != 0)
        return fail(MLA_ERR_UNSUPPORTED, "sparse_decode: an MXFP8 window needs dim + rope % 32 == 0");
    const bool win8 = win_ring && win_fmt == MLA_FMT_MXFP8;
    const float* sinks = epilogue ? epilogue->sinks : nullptr;
    const int32_t rope_dim = epilogue ? epilogue->rope_dim : 0;
    const float* rope_cs = epilogue ? epilogue->rope_cs : nullptr;
    if (sinks && !aligned(sinks, 4)) return fail(MLA_ERR_INVALID_ARG, "sparse_decode: misaligned sinks");
    if (rope_dim < 0 || (rope_dim > 0 && (!rope_cs || !aligned(rope_cs, 4))))
        return fail(MLA_ERR_INVALID_ARG, "sparse_decode: output RoPE needs rope_dim >= 0 and aligned rope_cs");
    if (rope_dim % 8 != 0 || rope_dim > d_v || rope_dim > 256)
        return fail(MLA_ERR_UNSUPPORTED, "sparse_decode: output RoPE needs rope_dim % 8 == 0, <= min(d_v, 256)");
    if (!aligned(q, 16) || !aligned(out, 16) || (win_ring && !win8 && !aligned(win_ring, 16)))
        return fail(MLA_ERR_INVALID_ARG, "sparse_decode: q, out and win_ring must be 16-byte aligned");
    if (!mla::decode_supported(main_row.fmt, main_row.dim, main_row.rope_dim, d_v, H))
        return fail(MLA_ERR_UNSUPPORTED, "sparse_decode: no kernel for this shape");
    const size_t base = mla::decode_workspace_bytes(main_row.fmt, main_row.dim, main_row.rope_dim, d_v, B, H, k,
                                                    win_ring ? W : 0);
    const size_t need = base + (win8 ? window_copy_bytes(win_fmt, B, W, D) : 0);
    if (base == 0 && (k + (win_ring ? W : 0) > 8192 || D > 1024))
        return fail(MLA_ERR_UNSUPPORTED, "sparse_decode: generic path limited to k + W <= 8192, width <= 1024");
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256)))
        return fail(MLA_ERR_WORKSPACE, "sparse_decode: workspace needs %zu bytes, 256-byte aligned", need);
    mla::DecodeArgs a{};
    a.fmt = main_row.fmt;
    a.dim = main_row.dim;
    a.rope = main_row.rope_dim;
    a.d_v = d_v;
    a.row_bytes = rb;
    a.q = q;
    a.cache = static_cast<const uint8_t*>(main_cache);
    a.stride = main_seq_stride;
    a.capacity = capacity;
    a.idx = idx;
    a.k = k;
    a.win = (win_ring && !win8) ? static_cast<const uint16_t*>(win_ring) : nullptr;
    a.win8 = win8 ? static_cast<const uint8_t*>(win_ring) : nullptr;
    a.win_len = win_len;
    a.W = win_ring ? W : 0;
    a.scale = softmax_scale;
    a.sinks = sinks;
    a.rope_dim = rope_dim;
    a.rope_cs = rope_cs;
    a.B = B;
    a.H = H;
    a.out = out;
    a.lse = lse;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    if (finish) {
        if (!mla::decode_takes_select_lists(a.fmt, a.dim, a.rope, a.d_v, B, H, k, a.W))
            return fail(MLA_ERR_UNSUPPORTED, "sparse_decode: this shape cannot finish a selection");
        a.idx = nullptr;
        a.sel_counts = sel->ws.counts;
        a.sel_lists = sel->ws.sel;
        a.cand_lists = sel->ws.cand;
        a.cand_flat = sel->ws.cand2;
        a.sel_hist = sel->ws.hist;
        a.sel_visible = sel->n_visible;
        a.sel_capacity = sel->capacity;
        a.sel_groups = sel->groups;
        a.idx_out = idx_out;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (new_win) {                                         // the step's window entry first
        a.new_win = new_win;
        a.win_pos = win_pos;
        if (!mla::decode_fuses_window_append(a)) {
            mla::AppendArgs ap{};
            const mla_status_t sa = append_args(main_row, mla_row_t{MLA_FMT_F32, 0, 0}, nullptr, nullptr, nullptr, B,
                                                0, capacity, nullptr, 0, nullptr, 0, new_win, win_pos,
                                                const_cast<void*>(win_ring), W, D, win_fmt, &ap);
            if (sa != MLA_OK) return sa;
            const hipError_t e = mla::launch_append(ap, st);
            if (e != hipSuccess) return hip_status(e, "window append launch");
            a.new_win = nullptr;
            a.win_pos = nullptr;
        }
    }
    return hip_status(mla::launch_decode(a, st), "sparse decode");
}

mla_status_t mla_sparse_decode(mla_row_t main_row, int32_t d_v, const void* q, const void* main_cache,
                               int64_t main_seq_stride, int64_t capacity, const int32_t* idx, int32_t k,
                               const void* win_ring, const int32_t* win_len, int32_t W, int32_t win_fmt,
                               float softmax_scale,
                               const mla_decode_epilogue_t* epilogue, int32_t B, int32_t H, float* out, float* lse,
                               void* workspace,
                               size_t workspace_bytes, void* stream) {
    mla::begin_call();
    return decode_impl(main_row, d_v, q, main_cache, main_seq_stride, capacity, idx, k, nullptr, nullptr, win_ring,
                       win_len, W, win_fmt, softmax_scale, epilogue, B, H, out, lse, workspace, workspace_bytes,
                       stream);
}

mla_status_t mla_append_sparse_decode(mla_row_t main_row, int32_t d_v, const void* q, const void* main_cache,
                                      int64_t main_seq_stride, int64_t capacity, const int32_t* idx, int32_t k,
                                      const float* new_win, const int32_t* win_pos, void* win_ring,
                                      const int32_t* win_len, int32_t W, int32_t win_fmt, float softmax_scale,
                                      const mla_decode_epilogue_t* epilogue, int32_t B, int32_t H, float* out,
                                      float* lse, void* workspace, size_t workspace_bytes, void* stream) {
    mla::begin_call();
    if (!new_win || !win_pos || !win_ring)
        return fail(MLA_ERR_INVALID_ARG, "append_sparse_decode: needs new_win, win_pos and win_ring");
    if (!aligned(new_win, 4) || !aligned(win_pos, 4))
        return fail(MLA_ERR_INVALID_ARG, "append_sparse_decode: misaligned new_win or win_pos");
    return decode_impl(main_row, d_v, q, main_cache, main_seq_stride, capacity, idx, k, new_win, win_pos, win_ring,
                       win_len, W, win_fmt, softmax_scale, epilogue, B, H, out, lse, workspace, workspace_bytes,
                       stream);
}

mla_status_t mla_sparse_decode_noalloc(mla_row_t main_row, int32_t d_v, const void* q, const void* main_cache,
                                       int64_t main_seq_stride, int64_t capacity, const int32_t* idx, int32_t k,
                                       const void* win_ring, const int32_t* win_len, int32_t W, int32_t win_fmt,
                                       float softmax_scale, const mla_decode_epilogue_t* epilogue, int32_t B,
                                       int32_t H, float* out, float* lse, void* stream) {
    mla::begin_call();
    const size_t need = (B > 0 && H > 0 && k >= 0 && W >= 0)
                            ? mla_sparse_decode_workspace(main_row, d_v, B, H, k, win_ring ? W : 0, win_fmt)
                            : 0;
    if (need > kScratchBytes)
        return fail(MLA_ERR_WORKSPACE, "sparse_decode_noalloc: this shape needs %zu bytes of scratch, above the "
                    "library's %zu", need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0 && !(ws = device_scratch())) return MLA_ERR_HIP;
    return mla_sparse_decode(main_row, d_v, q, main_cache, main_seq_stride, capacity, idx, k, win_ring, win_len, W,
                             win_fmt, softmax_scale, epilogue, B, H, out, lse, ws, ws ? kScratchBytes : 0, stream);
}


mla_status_t mla_csa2_group_step(mla_row_t main_row, mla_row_t idx_row, int32_t d_v, int32_t n_layers,
                                 const mla_group_layer_t* layers, const float* new_main, const float* new_idx,
                                 const int32_t* slots, int32_t n_new, void* main_cache, int64_t main_seq_stride,
                                 void* idx_cache, int64_t idx_seq_stride, int64_t capacity,
                                 const int32_t* n_visible, int32_t B, int32_t H, int32_t H_I, int32_t k,
                                 float score_scale, float softmax_scale, const int32_t* win_pos,
                                 const int32_t* win_len, int32_t W, int32_t win_fmt, int32_t score_bf16,
                                 int32_t pool_blocks, int32_t pool_block, float* pool_scores, int32_t* pool_pos,
                                 int32_t* idx_a, int32_t* idx_b, void* topk_workspace, size_t topk_workspace_bytes,
                                 void* decode_workspace, size_t decode_workspace_bytes, void* stream) {
    mla::begin_call();
    // the group's own arguments, every layer's, and the workspace sizes: checked before the
    // first launch (the calls below check the shared arguments again, identically each time)
    if (n_layers < 1 || !layers) return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: needs at least one layer");
    if (!idx_a || !idx_b || !aligned(idx_a, 4) || !aligned(idx_b, 4))
        return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: needs two 4-byte aligned index buffers");
    if (pool_blocks < 0 || (pool_blocks > 0 && (!pool_scores || !pool_pos)))
        return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: a pool needs pool_scores and pool_pos");
    bool selected = false;
    for (int32_t l = 0; l < n_layers; ++l) {
        const mla_group_layer_t& y = layers[l];
        if (y.mode != MLA_LAYER_FULL && y.mode != MLA_LAYER_REINDEX && y.mode != MLA_LAYER_REUSE)
            return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: layer %d has an unknown mode %d", l, y.mode);
        if (y.mode == MLA_LAYER_REUSE && !selected)
            return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: layer %d reuses indices no earlier layer selected", l);
        selected = true;
        if (!y.q || !y.out || !y.lse || !aligned(y.q, 16) || !aligned(y.out, 16) || !aligned(y.lse, 4))
            return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: layer %d needs q, out (16-byte aligned) and lse", l);
        if (y.mode != MLA_LAYER_REUSE && (!y.q_idx || !y.w || !aligned(y.q_idx, 16) || !aligned(y.w, 4)))
            return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: selecting layer %d needs q_idx (16-byte aligned) and w",
                        l);
        if (W > 0 && (!y.win_ring || !y.new_win || !aligned(y.win_ring, win_fmt == MLA_FMT_MXFP8 ? 2 : 16) ||
                      !aligned(y.new_win, 16)))
            return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: layer %d needs its window ring and entry (aligned)", l);
    }
    if (B < 0 || H < 1 || k < 0 || capacity < 0 || W < 0)
        return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: B, H, k, capacity or W out of range");
    const size_t need_topk = std::max(mla_indexer_topk_workspace(B, capacity, k),
                                      pool_blocks > 0 ? mla_indexer_pool_workspace(B, capacity, pool_block) : 0);
    if (!topk_workspace || topk_workspace_bytes < need_topk)
        return fail(MLA_ERR_WORKSPACE, "csa2_group_step: top-k workspace %zu bytes, needs %zu", topk_workspace_bytes,
                    need_topk);
    const size_t need_dec = mla_sparse_decode_workspace(main_row, d_v, B, H, k, W, win_fmt);
    if (need_dec > 0 && (!decode_workspace || decode_workspace_bytes < need_dec))
        return fail(MLA_ERR_WORKSPACE, "csa2_group_step: decode workspace %zu bytes, needs %zu",
                    decode_workspace_bytes, need_dec);

    struct Scope {                                         // one kernel record for the whole group
        Scope() { mla::group_begin(); }
        ~Scope() { mla::group_end(); }
    } scope;
    const int32_t Dw = main_row.dim + main_row.rope_dim;
    // a selecting layer's final folded into its decode: the many-workgroup selection over
    // every row (none with a pool, whose kernels reuse the top-k workspace), on the gather decode
    // (a Reindex layer scoring a pool keeps the final: its selection maps pool entries to positions;
    // a Full layer that publishes the pool does so after its decode, which reads the lists first)
    const bool fold = mla::decode_takes_select_lists(main_row.fmt, main_row.dim, main_row.rope_dim, d_v, B, H, k, W);
    if (W > 0 && n_layers > 1 && (!win_pos || !aligned(win_pos, 4)))
        return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: the window entries need win_pos (4-byte aligned)");
    if (W > 0 && (!win_len || !aligned(win_len, 4)))
        return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: a window needs win_len (4-byte aligned)");
    if (W > 0 && win_fmt != MLA_FMT_BF16 && win_fmt != MLA_FMT_MXFP8)
        return fail(MLA_ERR_UNSUPPORTED, "csa2_group_step: window entries must be BF16 or MXFP8");
    if (W > 0 && win_fmt == MLA_FMT_MXFP8 && Dw % 32 != 0)
        return fail(MLA_ERR_UNSUPPORTED, "csa2_group_step: an MXFP8 window needs dim + rope % 32 == 0");
    if (fold && B > 0 && k > 0) {                          // a decode that finishes a selection must not fail
        int64_t rb = 0;                                    // after it: its cache is checked first
        if (!main_cache) return fail(MLA_ERR_INVALID_ARG, "csa2_group_step: main_cache is NULL");
        const mla_status_t sc = check_rows("csa2_group_step", main_row, main_cache, main_seq_stride, capacity, B,
                                           &rb, true);
        if (sc != MLA_OK) return sc;
    }
    int32_t* bufs[2] = {idx_a, idx_b};
    int32_t* latest = nullptr;
    int j = 0;
    for (int32_t l = 0; l < n_layers; ++l) {
        const mla_group_layer_t& y = layers[l];
        mla_status_t st = MLA_OK;
        Deferred dfr;
        if (y.mode != MLA_LAYER_REUSE) {                   // full / reindex: select with the layer's own query
            latest = bufs[j % 2];
            float* scores = (pool_blocks > 0 && y.mode == MLA_LAYER_FULL) ? pool_scores : nullptr;
            if (l == 0) {                                  // carrying the step's append (and window entry)
                st = append_indexer_topk(
                    main_row, idx_row, new_main, new_idx, slots, n_new, new_main ? main_cache : nullptr,
                    main_seq_stride, idx_cache, idx_seq_stride, capacity, W > 0 ? y.new_win : nullptr,
                    W > 0 ? win_pos : nullptr, W > 0 ? y.win_ring : nullptr, W > 0 ? W : 0, W > 0 ? Dw : 0, win_fmt,
                    y.q_idx, y.w, score_scale, n_visible, B, H_I, k, latest, scores, topk_workspace,
                    topk_workspace_bytes, stream, score_bf16 != 0, fold ? &dfr : nullptr);
            } else {                                       // a Reindex layer with a pool scores the pool only
                const bool use_pool = pool_blocks > 0 && y.mode == MLA_LAYER_REINDEX;
                st = indexer_topk(idx_row, y.q_idx, y.w, score_scale, idx_cache, idx_seq_stride, capacity, n_visible,
                                  use_pool ? pool_pos : nullptr, use_pool ? pool_blocks * pool_block : 0, B, H_I, k,
                                  latest, scores, topk_workspace, topk_workspace_bytes, stream, score_bf16 != 0,
                                  fold ? &dfr : nullptr);
            }
            if (st == MLA_OK && scores && dfr.groups == 0)  // the Full layer publishes the candidate pool
                st = mla_indexer_pool(scores, capacity, n_visible, B, pool_block, pool_blocks, pool_pos,
                                      topk_workspace, topk_workspace_bytes, stream);
            if (st != MLA_OK) return st;
            ++j;
        }
        // (a deferred selection: the decode finishes it and writes the index set to `latest`)
        const Deferred* sel = dfr.groups > 0 ? &dfr : nullptr;
        if (l > 0 && W > 0)                                // the layer's window entry in its decode's call
            st = decode_impl(main_row, d_v, y.q, main_cache, main_seq_stride, capacity, latest, k, y.new_win, win_pos,
                             y.win_ring, win_len, W, win_fmt, softmax_scale, nullptr, B, H, y.out, y.lse,
                             decode_workspace, decode_workspace_bytes, stream, sel, latest);
        else
            st = decode_impl(main_row, d_v, y.q, main_cache, main_seq_stride, capacity, latest, k, nullptr, nullptr,
                             W > 0 ? y.win_ring : nullptr, W > 0 ? win_len : nullptr, W > 0 ? W : 0, win_fmt,
                             softmax_scale, nullptr, B, H, y.out, y.lse, decode_workspace, decode_workspace_bytes,
                             stream, sel, latest);
        if (st != MLA_OK) return st;
        if (sel && y.mode == MLA_LAYER_FULL && pool_blocks > 0)   // the pool, once the lists are read
            st = mla_indexer_pool(pool_scores, capacity, n_visible, B, pool_block, pool_blocks, pool_pos,
                                  topk_workspace, topk_workspace_bytes, stream);
        if (st != MLA_OK) return st;
    }
    return ok();
}

}  // extern "C"
