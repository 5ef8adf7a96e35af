// launch.hpp -- internal argument blocks and launchers of the gfx950 kernels.
// Host-side validation lives in api.cpp; launchers assume valid arguments.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <tuple>
#include <stdint.h>

namespace mla {

// Bins of the top-k score histogram (top 12 bits of the order-preserving key).
// Every sequence has kHistCopiesHost copies of a 64-bin coarse level (top 6 bits)
// followed by as many copies of the 4096-bin fine level; a scan workgroup adds
// into the copy its block index selects, so that no bin takes atomics from every
// workgroup of the sequence, and the selection sums the copies.
constexpr int kHistBinsHost = 4096;
constexpr int kHistCopiesHost = 8;
constexpr int kCoarseBinsHost = 64;
constexpr int64_t kHistWordsHost = (int64_t)kHistCopiesHost * (kCoarseBinsHost + kHistBinsHost);
// Work queues of the dynamic indexer scan, at the start of the top-k workspace:
// queue i's ticket counter is word kQueueWordsHost * i, its count of finished
// waves the word 16 after it (one 128-byte line per queue). Zero between calls.
constexpr int kScanQueuesHost = 512;
constexpr int kQueueWordsHost = 32;

struct AppendArgs {
    int main_fmt, main_dim, main_rope;
    int idx_fmt, idx_dim;
    int64_t main_row_bytes, idx_row_bytes;
    const float* new_main;
    const float* new_idx;
    const int32_t* slots;
    int B, n_new;
    int64_t capacity;
    uint8_t* main_cache;
    int64_t main_stride;
    uint8_t* idx_cache;
    int64_t idx_stride;
    const float* new_win;
    const int32_t* win_pos;
    uint16_t* win_ring;     // bf16 entries, or MXFP8 entries of Dw + Dw/32 bytes (win_fmt)
    int W, Dw;
    int win_fmt;
};
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);

// The CSA2 compressor at append (compress.hip).
struct CompressArgs {
    int fmt, dim, rope;     // main row format (D = dim + rope channels)
    int64_t row_bytes;
    const float* kv;        // [B, m, D]
    const float* gate;      // [B, m, D]
    const float* g;         // [D] normalisation weight, or null (ones)
    float eps;
    int m, D;
    int rope_dim;           // trailing channels rotated forward (0: none)
    const float* rope_cs;   // [B, rope_dim / 2, 2] (cos, sin)
    const int32_t* slots;   // [B] row of the entry, or null (no cache write)
    int64_t capacity;
    uint8_t* cache;
    int64_t stride;
    float* out;             // [B, D] fp32 entries, or null
    int B;
};
hipError_t launch_compress(const CompressArgs& a, hipStream_t stream);

// Workspace of the indexer + top-k, carved by the host (all 256-byte aligned).
struct TopkWorkspace {
    float* scores;          // [B, capacity] (used when the caller gives no score buffer)
    uint32_t* hist;         // [B, kHistWordsHost]: coarse [copies][64], then fine [copies][4096]
    uint32_t* counts;       // [B, select workgroups, 2]: each workgroup's selected / candidate count
    int32_t* sel;           // [B, capacity]: workgroup i's selected positions at i * kSelRowsHost ..
    uint64_t* cand;         // [B, capacity]: workgroup i's candidates (key << 32 | ~position) likewise
    uint64_t* cand2;        // [B, capacity]: all candidates of a sequence, contiguous
};
constexpr int kSelRowsHost = 2048;      // rows per select workgroup
inline int64_t select_groups(int64_t capacity) { return (capacity + kSelRowsHost - 1) / kSelRowsHost; }

struct ScanArgs {
    int fmt, dim;           // indexer row format
    int64_t row_bytes;
    const void* q_idx;      // [B, H_I, dim] bf16 (fp32 for F32 rows)
    const float* w;         // [B, H_I]
    float sigma;
    const uint8_t* cache;
    int64_t stride;
    int64_t capacity;
    const int32_t* n_visible;
    int B, H_I, k;
    float* scores;          // [B, capacity]
    uint32_t* hist;         // [B, kHistWordsHost] (see TopkWorkspace)
    uint32_t* queues;       // [kScanQueuesHost, kQueueWordsHost] work queues, zero on entry and on exit
    const int32_t* cand;    // [B, n_cand] positions of a candidate pool, or null: every row
    int64_t n_cand;         // pool entries per sequence; with a pool the scores are [B, n_cand] and
                            // the histogram counts every entry (those not visible as -inf)
    int score_bf16;         // 1: scores rounded to bf16 (round to nearest even) before they are
                            // stored, counted and selected (the bf16-score top-k)
};
// Entries of a step's append that the indexer scan can carry in the same launch.
constexpr int kFuseMaxNew = 4;
// The scan; with `append` (its cache the scan's, 1 <= n_new <= kFuseMaxNew), the
// quantise-append of the same step first, in the scan's launch where the scan
// kernel can carry it, else as its own launch before it.
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream, const AppendArgs* append = nullptr);
bool scan_supported(int fmt, int dim, int H_I);
// How the selection reports entry s of a sequence's scores: as s, or, with a
// candidate pool, as its position cand[b, s] (-1 when that is negative or not
// below min(n_visible[b], limit)); a reported value v is written as `expand`
// outputs v * expand + j (j < expand; -1 as -1s), so that a selection of blocks
// reports their positions.
struct SelectMap {
    const int32_t* cand = nullptr;      // [B, capacity]
    const int32_t* n_visible = nullptr;
    int64_t limit = 0;
    int expand = 1;
};
// The k largest of scores[b, 0 .. n_visible[b]) (every one of the capacity
// entries when n_visible is null) into out_idx [B, k * map.expand].
hipError_t launch_select(const float* scores, int64_t capacity, const int32_t* n_visible, int B, int k,
                         const TopkWorkspace& ws, int32_t* out_idx, hipStream_t stream,
                         const SelectMap& map = SelectMap{});
// k_select alone, when launch_select would take its many-workgroup path over every
// entry (no pool, no expansion) with at most kFusedSelectGroups workgroups per sequence:
// *groups = those workgroups, and the decode that follows finishes the selection from
// their lists (DecodeArgs.sel_*). Otherwise nothing is launched and *groups = 0.
constexpr int kFusedSelectGroups = 1024;
hipError_t launch_select_lists(const float* scores, int64_t capacity, const int32_t* n_visible, int B, int k,
                               const TopkWorkspace& ws, hipStream_t stream, int* groups);
// (the same from kFoldManyMin rows on, where the many-workgroup path with its final in the
// decode is ahead of the one-workgroup selection)
constexpr int64_t kFoldManyMin = 4096;
// Block maxima of a layer's scores ([B, capacity]): bmax[b, i] = the largest
// score among the visible positions block*i .. block*i + block - 1, the
// histogram of their keys into hist (as the scan builds it), and nvb[b] = the
// number of blocks holding a visible position.
hipError_t launch_block_max(const float* scores, int64_t capacity, const int32_t* n_visible, int B, int block,
                            float* bmax, int32_t* nvb, uint32_t* hist, hipStream_t stream);

struct DecodeArgs {
    int fmt, dim, rope, d_v;
    int64_t row_bytes;
    const void* q;          // [B, H, dim+rope] bf16 (fp32 for F32 rows)
    const uint8_t* cache;
    int64_t stride, capacity;
    const int32_t* idx;
    int k;
    const uint16_t* win;    // [B, W, dim+rope] bf16 or null
    const uint8_t* win8;    // or [B, W, D + D/32] MXFP8 entries (widened into the workspace first)
    const int32_t* win_len;
    int W;
    const float* new_win;   // [B, dim+rope] fp32: the step's window entry, written into ring slot
    const int32_t* win_pos; // win_pos[b] mod W by the decode itself (null: the ring is as given)
    float scale;
    const float* sinks;     // [H] attention-sink logits, or null
    int rope_dim;           // trailing output channels un-rotated (0: none)
    const float* rope_cs;   // [B, rope_dim / 2, 2] (cos, sin)
    int B, H;
    float* out;             // [B, H, d_v]
    float* lse;             // [B, H]
    void* workspace;
    size_t workspace_bytes;
    // A selection to finish (sel_counts null: the rows come from idx): k_select's lists of a
    // many-workgroup selection over scores [B, sel_capacity] (sel_groups workgroups per
    // sequence, each with its counts, selected positions and candidates), the histogram whose
    // rest is zeroed for the next call, and idx_out [B, k], where the decode writes the index
    // set the final would have written.
    const uint32_t* sel_counts = nullptr;
    const int32_t* sel_lists = nullptr;
    const uint64_t* cand_lists = nullptr;
    uint64_t* cand_flat = nullptr;          // [B, sel_capacity]: the candidates in one list, past LDS
    uint32_t* sel_hist = nullptr;
    const int32_t* sel_visible = nullptr;
    int64_t sel_capacity = 0;
    int sel_groups = 0;
    int32_t* idx_out = nullptr;
};
bool decode_supported(int fmt, int dim, int rope, int d_v, int H);
size_t decode_workspace_bytes(int fmt, int dim, int rope, int d_v, int B, int H, int k, int W);

// Opt-in per-kernel event timing (profile.cpp), off unless mla_profile_enable(1).
enum ProfKernel { PROF_APPEND, PROF_SCAN, PROF_SELECT, PROF_DECODE, PROF_MERGE, PROF_KERNELS };
struct ProfSlot {
    hipEvent_t start = nullptr, stop = nullptr;
};
ProfSlot prof_slot(ProfKernel k);  // a fresh event pair for one launch; two nulls while timing is off
void prof_enable(uint32_t mask);  // bit k times ProfKernel k
int prof_index(const char* name);  // -1 for an unknown name
hipError_t prof_read(int k, int32_t* launches, double* total_ms);

// Kernel-choice options (options.cpp; mla_set_option): 0 = the library's own choice.
enum Opt {
    OPT_TOPK_PATH, OPT_TOPK_FINAL, OPT_SCAN_QUEUES, OPT_SCAN_BLOCKS,
    OPT_DECODE_RPS, OPT_COUNT
};
int64_t option(Opt o);
int option_index(const char* name);     // -1 for an unknown name
bool option_set(int i, int64_t v);      // false when out of range
// The kernels the calling thread's current API call launches (mla_last_kernels).
void begin_call();
// Between these, the calls a group call makes add to one record (begin_call does not reset it).
void group_begin();
void group_end();
void note_launch(const void* f);
const char* launched_names();

// Launch `kernel`.  With events, through hipExtLaunchKernel: the runtime stamps
// them from the kernel's own dispatch (start, end), so a pair brackets exactly
// that kernel and no marker packet is added between kernels on the stream.
template <typename... Params, typename... Args>
hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block, uint32_t lds, hipStream_t stream,
                         hipEvent_t t0, hipEvent_t t1, Args... args) {
    static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
    std::tuple<Params...> held{args...};
    void* argv[sizeof...(Params)];
    std::apply([&](auto&... x) {
        int i = 0;
        ((argv[i++] = static_cast<void*>(&x)), ...);
    }, held);
    const void* f = reinterpret_cast<const void*>(kernel);
    note_launch(f);
    if (t0 || t1) return hipExtLaunchKernel(f, grid, block, argv, lds, stream, t0, t1, 0);
    return hipLaunchKernel(f, grid, block, argv, lds, stream);
}
size_t decode_workspace_bytes(int fmt, int dim, int rope, int d_v, int B, int H, int k, int W);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Whether launch_decode can finish a selection from k_select's lists for this shape
// (the MFMA decodes; W: window slots, 0 without a window).
bool decode_takes_select_lists(int fmt, int dim, int rope, int d_v, int B, int H, int k, int W);
// Whether launch_decode writes a.new_win into the window ring itself (512-channel bf16 or
// MXFP8 entries on the gather decode); otherwise the caller appends it first.
bool decode_fuses_window_append(const DecodeArgs& a);

}  // namespace mla
