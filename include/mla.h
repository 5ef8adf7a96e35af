/*
 * mla.h -- C ABI of the MI355X (gfx950) decode hot path for indexer-selected
 * sparse attention over a block-scaled latent KV cache.
 *
 * One decode step of one layer is three calls:
 *   mla_kv_append_quant   quantise the new entry (and indexer key) into the caches,
 *                         write the window ring;
 *   mla_indexer_topk      lightning-indexer scan over the indexer keys, causal mask,
 *                         top-k -> int32 positions;
 *   mla_sparse_decode     absorbed-MLA attention over the selected entries (plus the
 *                         window), online softmax, logsumexp output.
 * mla_append_indexer_topk is the first two in one call (the append then rides in
 * the scan's launch where the scan kernel can carry it).  mla_indexer_pool turns
 * one layer's scores into the candidate pool of the hierarchical sparse indexer,
 * which deeper layers' mla_indexer_topk calls then score instead of every row.
 * The cross-layer sharing modes of CSA2 are compositions of these calls over
 * shared pointers: Full = append + topk + decode; Reindex = topk with its own
 * indexer query over another layer's indexer cache + decode over the shared main
 * cache; Reuse = decode with the shared indices.  mla_csa2_group_step enqueues a
 * whole group's calls in one call from C.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "DeepSeek's Attention and KV Cache - From MLA to CSA2, From First Principles"
 *  [P2] "From MLA to DSA to HCA/CSA: DeepSeek V3.2 and V4 Attention"
 *  [P3] "DeepSeek-V4.1-Flash and the 890-byte KV cache"
 *  [P4] "From First Principles: DeepSeek-V4.1-Flash Inference"
 *
 * Conventions common to every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller; the library
 *    allocates nothing and keeps no state beyond a thread-local error string.
 *  - `stream` is a hipStream_t passed as void*; calls only enqueue kernels on
 *    it and never synchronise.  NULL means the default stream.
 *  - Arguments are validated on the host before any launch; a call that
 *    returns an error has enqueued nothing (except MLA_ERR_HIP, where a launch
 *    itself failed).  mla_last_error() then holds a message.
 *  - Byte strides are int64; rows are little-endian byte arrays.  A cache's base
 *    pointer must be 16-byte aligned and its sequence stride a multiple of the
 *    row alignment (the largest power of two <= 16 dividing the row size:
 *    16 for 656 / 288 / 256-byte rows, 8 for 72, 4 for 132).
 *  - Non-finite inputs give unspecified (but memory-safe) results.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARG = 1,   /* null required pointer, bad size, bad stride, misalignment */
    MLA_ERR_UNSUPPORTED = 2,   /* a format / shape combination with no kernel */
    MLA_ERR_WORKSPACE = 3,     /* workspace missing or too small */
    MLA_ERR_HIP = 4            /* a HIP launch or runtime call failed */
} mla_status_t;

/* Row formats of a cached entry.
 *  MLA_FMT_F32       (dim+rope) fp32 values.
 *  MLA_FMT_BF16      (dim+rope) bf16 values.
 *  MLA_FMT_E4M3_S128 [dim E4M3 codes | dim/128 fp32 scales | rope bf16]; dim % 128 == 0.
 *                    V3.2: 512 + 16 + 128 = 656 B main row, 128 + 4 = 132 B indexer
 *                    key ([P1] "DeepSeek-V3.2", "What it costs and what it saves").
 *                    Scale of a 128-channel block: amax/448 in fp32; code = E4M3
 *                    round-to-nearest-even of x/scale (fp32 division), saturating.
 *  MLA_FMT_E2M1_S16  [dim/2 bytes of E2M1 nibbles, channel 2i in the low nibble of
 *                    byte i | dim/16 E4M3 scale bytes]; dim % 16 == 0, rope == 0.
 *                    V4.1: 256 + 32 = 288 B main row ([P1] "DeepSeek-V4.1", "Four
 *                    bits for the main KV"); 64 + 8 = 72 B indexer key ([P3] section 3).
 *                    Scale of a 16-channel block: E4M3(amax / 6) (fp32 division,
 *                    round-to-nearest-even, saturating); code = E2M1 nearest-even of
 *                    x/scale; a zero scale gives zero codes.
 *  MLA_FMT_MXFP4     [dim/2 bytes of E2M1 nibbles as above | dim/32 E8M0 scale bytes];
 *                    dim % 32 == 0, rope == 0. V4's indexer keys: 64 + 4 = 68 B
 *                    ([P1] "DeepSeek-V4", "The indexer in four bits"; [P4] "FP4 main
 *                    KV: smaller cells"). The OCP microscaling rule: the E8M0 code of a
 *                    32-channel block is floor(log2 amax) - 2 + 127, clamped to 0..254
 *                    (0 for a block of zeros), its scale X = 2^(code - 127); code =
 *                    E2M1 nearest-even of x/X, saturating at 6. As an indexer format it
 *                    makes the query-key product FP4 on both sides: mla_indexer_topk
 *                    rounds each head's query to MXFP4 the same way before scoring.
 *  MLA_FMT_MXFP8     [dim E4M3 codes | dim/32 E8M0 scale bytes]; dim % 32 == 0, rope == 0;
 *                    window entries only (win_fmt below): V4.1's 512 + 16 = 528 B window
 *                    entry ([P1] "DeepSeek-V4.1"). The same OCP rule with E4M3's largest
 *                    exponent: code floor(log2 amax) - 8 + 127, clamped to 0..254 (0 for a
 *                    block of zeros); element = E4M3 nearest-even of x/X, saturating at 448.
 * E4M3 is the OCP "fn" variant (max 448, no infinities); E2M1 magnitudes are
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 ([P1] "A Precision Primer"); an E8M0 code e is 2^(e - 127). */
typedef enum {
    MLA_FMT_F32 = 0,
    MLA_FMT_BF16 = 1,
    MLA_FMT_E4M3_S128 = 2,
    MLA_FMT_E2M1_S16 = 3,
    MLA_FMT_MXFP4 = 4,
    MLA_FMT_MXFP8 = 5
} mla_fmt_t;

/* A row: `dim` quantised (or plain) channels followed by `rope_dim` RoPE channels.
 * The attention key of a main row is all dim+rope channels ([c_KV ; k_R] of the
 * absorbed form, [P1] "DeepSeek-V2", "Why RoPE breaks the trick"). */
typedef struct {
    int32_t dim;
    int32_t rope_dim;
    int32_t fmt;          /* an mla_fmt_t */
} mla_row_t;

/* Bytes of one row, or -1 if the format / shape is not supported. */
int64_t mla_row_bytes(mla_row_t row);

/* Static text of a status code. */
const char* mla_status_str(int32_t status);

/* Detail of the last error on the calling thread ("" if none). */
const char* mla_last_error(void);

/* ABI version (major * 100 + minor). */
int32_t mla_version(void);

/*
 * Measurement hooks (not part of the computation). mla_profile_enable(mask)
 * selects kernels to time; each later launch of a selected kernel takes a pair
 * of HIP events that the runtime stamps from that kernel's own dispatch
 * (hipExtLaunchKernel), on the caller's stream, so the pair measures exactly
 * the kernel's execution. Timed launches cost more host time than plain ones.
 * mask 0 (the default) times nothing; MLA_PROF_ALL times all of them.
 * mla_profile_read waits for the recorded pairs of one kernel, returns how many
 * there were and their summed duration in milliseconds, and starts a new count.
 *   bit  name
 *   0    "kv_append"     the kernel of mla_kv_append_quant
 *   1    "indexer_scan"  the indexer scan of mla_indexer_topk
 *   2    "topk_select"   its top-k selection (one kernel, or the first's start
 *                        to the second's end)
 *   3    "decode"        the split attention kernel of mla_sparse_decode
 *   4    "decode_merge"  its logsumexp merge
 * Events are created on first use and kept for reuse; taking them is
 * serialised by a lock. Errors: MLA_ERR_INVALID_ARG (unknown name, NULL
 * pointer), MLA_ERR_HIP (an event query failed).
 */
#define MLA_PROF_KV_APPEND 0x01
#define MLA_PROF_INDEXER_SCAN 0x02
#define MLA_PROF_TOPK_SELECT 0x04
#define MLA_PROF_DECODE 0x08
#define MLA_PROF_DECODE_MERGE 0x10
#define MLA_PROF_ALL 0x1f
mla_status_t mla_profile_enable(int32_t kernels);
mla_status_t mla_profile_read(const char* kernel, int32_t* launches, double* total_ms);

/*
 * Kernel-choice options (process-wide; not part of the computation). Several
 * calls have more than one kernel that computes the same result; by default
 * (every option 0) the library picks by shape. An option forces a choice, for
 * tuning and for tests that must reach a particular kernel. Options are read at
 * each call, so set them before the calls they should affect and not while
 * another thread is calling.
 *   name                     range      meaning of a non-zero value
 *   "topk_path"              0..2       1: one workgroup selects each sequence;
 *                                       2: many select workgroups and a final step
 *   "topk_final"             0..1       1: the 256-thread final of the many-workgroup path
 *   "scan_queues"            0..1       1: the queue-fed 32x32 indexer scan
 *   "scan_blocks"            0..65536   target number of 4-wave indexer-scan workgroups
 *   "decode_rows_per_split"  0..256     selected rows per decode split (a multiple of 32 up to
 *                                       256 for E4M3 rows, 128 for E2M1 rows and bf16 rows
 *                                       decoded 16 heads per workgroup; a multiple of 64 from
 *                                       64 for bf16 rows decoded 32 heads per workgroup)
 * Values in range that a kernel cannot use are ignored. Errors:
 * MLA_ERR_INVALID_ARG (unknown name, NULL pointer, value out of range).
 */
mla_status_t mla_set_option(const char* name, int64_t value);
mla_status_t mla_get_option(const char* name, int64_t* value);

/*
 * The kernels that the calling thread's most recent compute call (append,
 * compress, top-k, pool or decode) launched, as demangled names separated by
 * ';' ("" if it launched none). Valid until the thread's next call of this
 * function. For tests and tuning: it shows which kernel served a call.
 */
const char* mla_last_kernels(void);

/*
 * mla_kv_append_quant -- quantise-append of one decode step's entries.
 *
 * Writes, for each sequence b and each new entry i < n_new, the quantised main
 * row of new_main[b, i, :] into main_cache at row slots[b, i], and the quantised
 * indexer key of new_idx[b, i, :] into idx_cache at the same row.  The entry is
 * quantised after RoPE, with no global scale ([P1] "DeepSeek-V4.1", "Four bits
 * for the main KV"); the indexer key uses its own row format.  If new_win is
 * given, the bf16 (round-to-nearest-even) window entry new_win[b, :] is written
 * to ring slot win_pos[b] mod W ([P1] "Sliding Window Attention", "Definition and
 * the bounded cache").
 *
 *  main_row, idx_row  row formats (idx_row.rope_dim must be 0)
 *  new_main           fp32 [B, n_new, main.dim + main.rope_dim]; may be NULL iff main_cache is NULL
 *  new_idx            fp32 [B, n_new, idx.dim]; may be NULL iff idx_cache is NULL
 *  slots              int32 [B, n_new], each in [0, capacity); required if either cache is given
 *  capacity           rows allocated per sequence (checked against slots on the device:
 *                     out-of-range slots are skipped, not written)
 *  main_cache         bytes, row r of sequence b at b*main_seq_stride + r*row_bytes; or NULL
 *  idx_cache          likewise for indexer keys; or NULL
 *  new_win            fp32 [B, Dw] or NULL (no window write)
 *  win_pos            int32 [B] absolute positions (>= 0) of the window entries
 *  win_ring           [B, W, entry bytes]: bf16 [B, W, Dw] (win_fmt MLA_FMT_BF16) or
 *                     MXFP8 entries of Dw + Dw/32 bytes (win_fmt MLA_FMT_MXFP8, Dw % 32 == 0,
 *                     Dw <= 2048: the 528-byte window entry of V4.1 at Dw = 512)
 *  win_fmt            MLA_FMT_BF16 or MLA_FMT_MXFP8 (ignored without a window)
 * Errors: MLA_ERR_INVALID_ARG for B < 0, n_new < 0, missing pointers, strides
 * smaller than capacity * row_bytes, W <= 0 or Dw <= 0 with a window;
 * MLA_ERR_UNSUPPORTED for an unsupported row format.
 */
mla_status_t mla_kv_append_quant(mla_row_t main_row, mla_row_t idx_row,
                                 const float* new_main, const float* new_idx,
                                 const int32_t* slots, int32_t B, int32_t n_new, int64_t capacity,
                                 void* main_cache, int64_t main_seq_stride,
                                 void* idx_cache, int64_t idx_seq_stride,
                                 const float* new_win, const int32_t* win_pos,
                                 void* win_ring, int32_t W, int32_t Dw, int32_t win_fmt,
                                 void* stream);

/*
 * mla_compress_append -- the CSA2 compressor at append, fused with the quantise-append.
 *
 * V4.1 pools each window of m tokens into one cache entry, the windows not
 * overlapping and with no position bias ([P1] "DeepSeek-V4.1", "CSA2: the
 * simplified compressor"; [P2] Part 2, the compressor's training-path code).
 * For each sequence b, from the projected kv[b, i, :] and gate[b, i, :] of the
 * window's tokens i < m (D = main_row.dim + main_row.rope_dim channels):
 *     w[i, c] = softmax over i of gate[i, c]        p[c] = sum_i w[i, c] kv[i, c]
 *     y[c]    = p[c] / sqrt(mean_c p[c]^2 + eps) * norm_weight[c]
 * then, with rope_dim r > 0, the trailing r channels are rotated forward at the
 * window's position (rotate-half pairing: x1 = y[D-r .. D-r/2), x2 = y[D-r/2 .. D),
 * pair i becomes (x1 cos - x2 sin, x2 cos + x1 sin), (cos, sin) = rope_cs[b, i]),
 * and y is quantised into main_cache at row slots[b] exactly as mla_kv_append_quant
 * quantises an entry. The kv / gate projections and the indexer key's projection
 * from the entry are the caller's matmuls; out_entry returns y in fp32 for the latter.
 *
 *  kv, gate           fp32 [B, m, D], m >= 1
 *  norm_weight        fp32 [D], or NULL (ones); eps >= 0
 *  rope_dim, rope_cs  0 / NULL, or r even, r <= min(D, 512), with fp32 [B, r/2, 2] (cos, sin)
 *  slots              int32 [B] rows in [0, capacity) (others are skipped); NULL with
 *                     main_cache NULL (no cache write)
 *  main_cache         rows as in mla_kv_append_quant, or NULL; main_seq_stride its stride
 *  out_entry          fp32 [B, D], or NULL
 * Works in fp32 (the softmax online over the tokens). D <= 2048.
 * Errors: MLA_ERR_INVALID_ARG for negative sizes, missing pointers, m < 1, eps < 0,
 * an odd or too large rope_dim; MLA_ERR_UNSUPPORTED for an unsupported row or D > 2048.
 */
mla_status_t mla_compress_append(mla_row_t main_row, const float* kv, const float* gate, int32_t m,
                                 const float* norm_weight, float eps, int32_t rope_dim, const float* rope_cs,
                                 const int32_t* slots, int32_t B, int64_t capacity,
                                 void* main_cache, int64_t main_seq_stride, float* out_entry, void* stream);

/*
 * mla_indexer_topk -- lightning-indexer scan, causal mask and top-k.
 *
 * For every sequence b and cached row s < n_visible[b]:
 *     I[b, s] = sum_j w[b, j] * ReLU(score_scale * q_idx[b, j, :] . k_idx[b, s, :])
 * with one shared indexer key per row ([P1] "DeepSeek-V3.2", "The lightning
 * indexer", eq. 1; [P2] Part 1, "The indexer"), accumulated in fp32.  Rows at or
 * beyond n_visible[b] are masked ([P2] Part 2 "HCA": entry e is visible to query
 * position p iff e < (p + 1) // m).  The k visible rows of largest score are
 * returned as positions ([P1] eq. 2; ties at the k-th score go to the smaller
 * position); slots past min(k, n_visible[b]) hold -1 ([P2] "CSA: two changes to
 * HCA").  The returned positions are an unordered set.
 *
 *  idx_row      indexer-key row format (rope_dim 0)
 *  q_idx        [B, H_I, idx_row.dim] bf16, or fp32 when idx_row.fmt == MLA_FMT_F32
 *  w            fp32 [B, H_I], the per-head weights already scaled by the caller
 *               (the V3.2 code multiplies them by H_I^-0.5)
 *  score_scale  sigma > 0 applied inside the ReLU (d_I^-0.5 in the V3.2 code)
 *  idx_cache    indexer rows, row s of sequence b at b*idx_seq_stride + s*row_bytes;
 *               idx_seq_stride 0 makes every batch row read the same sequence: several
 *               queries of one sequence in one call (multi-token prediction), each with its
 *               own q_idx, w and n_visible (its causal limit)
 *  capacity     rows allocated per sequence (the scan covers rows < n_visible[b] <= capacity)
 *  n_visible    int32 [B] on the device, each in [0, capacity]
 *  cand, n_cand NULL and 0: every row is a candidate.  Otherwise a candidate pool
 *               ([P4] "The Hierarchical Sparse Indexer: bounded sweeps"; [P1]
 *               "DeepSeek-V4.1", "The hierarchical indexer": a Reindex layer scores
 *               only the positions a Full layer published, e.g. by
 *               mla_indexer_pool): int32 [B, n_cand] positions, n_cand >= 0, on the
 *               device.  Only the pool's positions are scored; an entry that is
 *               negative or not below n_visible[b] is never selected (its score is
 *               -inf).  The positions of one sequence's pool must be distinct.
 *               The selection is over the pool's visible positions with the same
 *               order and tie rule, and out_idx holds positions as without a pool.
 *  out_idx      int32 [B, k]
 *  out_scores   optional fp32 [B, capacity], or [B, n_cand] with a pool (entry i =
 *               the score of position cand[b, i]): the scores, -inf for masked rows
 *  workspace    device scratch of at least mla_indexer_topk_workspace(B, R, k) bytes,
 *               R = capacity (with a pool: the larger of capacity and n_cand),
 *               256-byte aligned, ZEROED BEFORE ITS FIRST USE (e.g. hipMemset once
 *               after allocation). It holds the scan's work-queue counters and the score
 *               histogram at its start; every call
 *               that returns MLA_OK leaves that part zeroed again, so one workspace serves
 *               any sequence of calls (any B, capacity, k within its size). A call that
 *               fails with MLA_ERR_HIP may leave it dirty: zero it again. Calls that
 *               share a workspace must not overlap in time (one stream, or ordered).
 * Errors: MLA_ERR_INVALID_ARG (pointers, B < 0, H_I < 1, k < 0, capacity < 0,
 * n_cand < 0 or n_cand > 0 without cand, score_scale <= 0, misalignment),
 * MLA_ERR_UNSUPPORTED (format / H_I / dim with no kernel), MLA_ERR_WORKSPACE.
 */
size_t mla_indexer_topk_workspace(int32_t B, int64_t capacity, int32_t k);

mla_status_t mla_indexer_topk(mla_row_t idx_row, const void* q_idx, const float* w,
                              float score_scale,
                              const void* idx_cache, int64_t idx_seq_stride, int64_t capacity,
                              const int32_t* n_visible,
                              const int32_t* cand, int32_t n_cand,
                              int32_t B, int32_t H_I, int32_t k,
                              int32_t* out_idx, float* out_scores,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_indexer_topk_bf16 -- the bf16-score top-k.
 *
 * mla_indexer_topk with every score rounded to bf16 (round to nearest even;
 * -inf stays -inf) before it is stored, counted and selected: the selection
 * is the k visible rows of largest bf16 score, ties -- now frequent: bf16 keeps
 * 8 significant bits -- going to the smaller position ([P1] "DeepSeek-V4", "The
 * indexer in four bits": index scores in bf16 instead of fp32). out_scores, if
 * given, receives the rounded scores as fp32 values (each exactly a bf16 value).
 * Same arguments, workspace and errors as mla_indexer_topk.
 */
mla_status_t mla_indexer_topk_bf16(mla_row_t idx_row, const void* q_idx, const float* w,
                                   float score_scale,
                                   const void* idx_cache, int64_t idx_seq_stride, int64_t capacity,
                                   const int32_t* n_visible,
                                   const int32_t* cand, int32_t n_cand,
                                   int32_t B, int32_t H_I, int32_t k,
                                   int32_t* out_idx, float* out_scores,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_indexer_pool -- the candidate pool of the hierarchical sparse indexer.
 *
 * From one layer's indexer scores ([P4] "The Hierarchical Sparse Indexer:
 * bounded sweeps"; [P1] "DeepSeek-V4.1", "The hierarchical indexer"): the positions of
 * sequence b are grouped into blocks of `block` consecutive positions (block i =
 * positions block*i .. block*i + block - 1), each block holding a visible position
 * is scored by the largest score among its visible positions, and the n_blocks
 * best blocks are kept (order by block score descending, ties to the smaller
 * block index, as in mla_indexer_topk).  out_pos[b] receives the positions of the
 * kept blocks, block*i + j for j < block in slots block*m .. block*m + block - 1 of
 * the m-th kept block (the order of the blocks is unspecified); the block slots
 * past min(n_blocks, blocks with a visible position) hold -1.  A kept partial last
 * block also lists its positions at or past n_visible[b]: mla_indexer_topk never
 * selects them.  V4.1 publishes 2,048 blocks of 8 (16,384 positions).
 *
 *  scores     fp32 [B, capacity] on the device, e.g. the out_scores of the layer's
 *             own mla_indexer_topk call; entries at or past n_visible[b] are not read
 *  n_visible  int32 [B], each in [0, capacity]
 *  block      a power of two, 1 .. 64 (block 1 gives the top-n_blocks positions)
 *  n_blocks   blocks kept per sequence (>= 0)
 *  out_pos    int32 [B, n_blocks * block]
 *  workspace  at least mla_indexer_pool_workspace(B, capacity, block) bytes,
 *             256-byte aligned, under the same zeroing contract as the workspace
 *             of mla_indexer_topk (the two may share one buffer that is large
 *             enough for both, used by one call at a time)
 * Errors: MLA_ERR_INVALID_ARG (pointers, B < 0, capacity < 0, n_blocks < 0,
 * misalignment), MLA_ERR_UNSUPPORTED (block not a power of two <= 64, sizes at or
 * over 2^31), MLA_ERR_WORKSPACE.
 */
size_t mla_indexer_pool_workspace(int32_t B, int64_t capacity, int32_t block);

mla_status_t mla_indexer_pool(const float* scores, int64_t capacity, const int32_t* n_visible,
                              int32_t B, int32_t block, int32_t n_blocks, int32_t* out_pos,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_append_indexer_topk -- one step's quantise-append followed by its indexer
 * top-k, in one call.
 *
 * Exactly mla_kv_append_quant(main_row, idx_row, new_main, new_idx, slots, B,
 * n_new, capacity, main_cache, main_seq_stride, idx_cache, idx_seq_stride,
 * new_win, win_pos, win_ring, W, Dw) and then mla_indexer_topk(idx_row, q_idx,
 * w, score_scale, idx_cache, idx_seq_stride, capacity, n_visible, NULL, 0, B,
 * H_I, k, out_idx, out_scores, workspace, workspace_bytes) on the same stream:
 * same arguments, same results and the same errors, the new indexer keys scored
 * from the bytes the append writes ([P1] "DeepSeek-V3.2", "The lightning
 * indexer": the step's own entry is among the keys its query ranks). Where
 * the scan kernel can carry it (E4M3 or E2M1 indexer rows of 128 channels, 32
 * or 64 indexer heads, 16-byte aligned cache, 1 <= n_new <= 4) the append runs
 * inside the scan's launch, which saves a launch and its memory round trip;
 * otherwise it is launched first, as its own kernel. idx_cache must not be
 * NULL; main_cache may be (indexer key and window only). The slots of one
 * sequence must be distinct.
 */
mla_status_t mla_append_indexer_topk(mla_row_t main_row, mla_row_t idx_row,
                                     const float* new_main, const float* new_idx,
                                     const int32_t* slots, int32_t n_new,
                                     void* main_cache, int64_t main_seq_stride,
                                     void* idx_cache, int64_t idx_seq_stride, int64_t capacity,
                                     const float* new_win, const int32_t* win_pos,
                                     void* win_ring, int32_t W, int32_t Dw, int32_t win_fmt,
                                     const void* q_idx, const float* w, float score_scale,
                                     const int32_t* n_visible, int32_t B, int32_t H_I, int32_t k,
                                     int32_t* out_idx, float* out_scores,
                                     void* workspace, size_t workspace_bytes, void* stream);

/* mla_append_indexer_topk_bf16 -- mla_append_indexer_topk whose top-k is the bf16-score
 * top-k of mla_indexer_topk_bf16 (same arguments and errors). */
mla_status_t mla_append_indexer_topk_bf16(mla_row_t main_row, mla_row_t idx_row,
                                          const float* new_main, const float* new_idx,
                                          const int32_t* slots, int32_t n_new,
                                          void* main_cache, int64_t main_seq_stride,
                                          void* idx_cache, int64_t idx_seq_stride, int64_t capacity,
                                          const float* new_win, const int32_t* win_pos,
                                          void* win_ring, int32_t W, int32_t Dw, int32_t win_fmt,
                                          const void* q_idx, const float* w, float score_scale,
                                          const int32_t* n_visible, int32_t B, int32_t H_I, int32_t k,
                                          int32_t* out_idx, float* out_scores,
                                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_sparse_decode -- absorbed MLA as shared-KV MQA over the selected entries.
 *
 * For each (b, h), over the multiset U = {rows idx[b, i] != -1} plus the window
 * slots 0 .. win_len[b]-1 (concatenated, not de-duplicated: [P1] "DeepSeek-V4",
 * "A window in every layer"):
 *     z_u   = softmax_scale * q[b, h, :] . K_u          (K_u = all dim+rope channels)
 *     lse   = logsumexp_u z_u                          (natural log)
 *     out   = sum_u exp(z_u - lse) * K_u[0 : d_v]       (V = the leading d_v channels)
 * This is the absorbed form ([P1] "DeepSeek-V2", "Check it in numpy"; [P2] Part 2,
 * "What replaced MLA"): q is the query with W_UK already folded in, the output is
 * the latent before W_UV.  Each selected row is read once for all heads ([P1]
 * "DeepSeek-V3.2").  An empty U gives lse = -inf and out = 0.
 *
 *  main_row    main row format; d_v <= dim
 *  q           [B, H, dim+rope] bf16 (fp32 when main_row.fmt == MLA_FMT_F32)
 *  main_cache  rows as in mla_kv_append_quant; capacity rows per sequence; main_seq_stride
 *              0 makes every batch row read the same sequence (several queries of one
 *              sequence, each with its own q, idx and window rows)
 *  idx         int32 [B, k]: positions in [0, capacity) or -1 (skipped); duplicates
 *              are attended twice
 *  win_ring    optional window entries (K = V) in format win_fmt: bf16 [B, W, dim+rope]
 *              (16-byte aligned) or MXFP8 [B, W, D + D/32] bytes (D = dim+rope, D % 32 ==
 *              0), widened to bf16 (exact for every block whose scale code is at least 3):
 *              512-channel entries in a 16-byte aligned ring as the decode stages them,
 *              others into the workspace by a launch of their own first, with
 *  win_len     int32 [B] in [0, W], the number of valid ring slots (slots 0..len-1)
 *  epilogue    optional (NULL = none):
 *              sinks: fp32 [H] attention-sink logits, one per head, shared by the batch
 *              ([P2] Part 2 "The sliding window", "Attention sinks": an extra score column
 *              with no value vector), in the units of the scaled scores z. With sinks,
 *              lse = log(sum_u exp(z_u) + exp(sinks[h])) and out = sum_u exp(z_u - lse)
 *              K_u[0 : d_v] (the weights of U sum to 1 - p_sink); an empty U gives lse =
 *              sinks[h] and out = 0.
 *              rope_dim, rope_cs: the output's RoPE inverse ([P2] Part 2 "What replaced
 *              MLA", "Partial RoPE, and its inverse on the output": K = V carries the
 *              rotation, which V4 undoes at the query position): with halves x1 =
 *              out[d_v - r .. d_v - r/2) and x2 = out[d_v - r/2 .. d_v), pair i becomes
 *              (x1 cos + x2 sin, x2 cos - x1 sin) with (cos, sin) = rope_cs[b, i].
 *  out         fp32 [B, H, d_v];  lse fp32 [B, H]
 *  workspace   at least mla_sparse_decode_workspace(main_row, d_v, B, H, k, W) bytes,
 *              256-byte aligned
 * Positions outside [0, capacity) other than -1 are skipped.
 * Errors: MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE.
 */
/* Optional epilogue of mla_sparse_decode: the V4 output path. */
typedef struct {
    const float* sinks;     /* [H] attention-sink logits (see mla_sparse_decode), or NULL */
    int32_t rope_dim;       /* 0, or r trailing output channels to un-rotate (r % 8 == 0, r <= min(d_v, 256)) */
    const float* rope_cs;   /* [B, r / 2, 2]: (cos, sin) of each sequence's query position, per RoPE pair */
} mla_decode_epilogue_t;

size_t mla_sparse_decode_workspace(mla_row_t main_row, int32_t d_v, int32_t B, int32_t H,
                                   int32_t k, int32_t W, int32_t win_fmt);

mla_status_t mla_sparse_decode(mla_row_t main_row, int32_t d_v, const void* q,
                               const void* main_cache, int64_t main_seq_stride, int64_t capacity,
                               const int32_t* idx, int32_t k,
                               const void* win_ring, const int32_t* win_len, int32_t W, int32_t win_fmt,
                               float softmax_scale, const mla_decode_epilogue_t* epilogue, int32_t B, int32_t H,
                               float* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * mla_append_sparse_decode -- the step's window entry appended, then the decode, in
 * one call ([P1] "DeepSeek-V4", "A window in every layer": every layer writes the
 * step's own entry into its window, then attends over the window and its selected
 * rows; [P1] "DeepSeek-V4.1", "Three modes": a Reuse layer's step is exactly this).
 *
 * Exactly mla_kv_append_quant(window entry only: new_win, win_pos, win_ring, W, Dw =
 * dim + rope, win_fmt) followed by mla_sparse_decode with the same ring, on the same
 * stream: afterwards the ring holds the entry's bytes in slot win_pos[b] mod W
 * (win_pos[b] < 0: sequence b appends nothing), and the decode attends over them.
 * With 512-channel bf16 or MXFP8 entries (16-byte aligned ring and new_win) on the
 * gather decode, the decode's window split writes the entry itself and stages it from
 * new_win, with no launch of its own; otherwise the append is launched first.
 *  new_win   fp32 [B, dim + rope], device
 *  win_pos   int32 [B] positions, device
 *  win_ring  the ring, writable; the other arguments, the workspace and the errors as
 *            for mla_sparse_decode (win_ring, win_len and W > 0 are required).
 */
mla_status_t mla_append_sparse_decode(mla_row_t main_row, int32_t d_v, const void* q,
                                      const void* main_cache, int64_t main_seq_stride, int64_t capacity,
                                      const int32_t* idx, int32_t k, const float* new_win,
                                      const int32_t* win_pos, void* win_ring, const int32_t* win_len,
                                      int32_t W, int32_t win_fmt, float softmax_scale,
                                      const mla_decode_epilogue_t* epilogue, int32_t B, int32_t H,
                                      float* out, float* lse, void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * mla_csa2_group_step -- one decode step of a layer group over one shared cache, in one call.
 *
 * The layers of a CSA2 group ([P1] "DeepSeek-V4.1", "Three modes"; [P4] "CSA2: four layers
 * keep their own copy") enqueued in order on `stream`, each as the calls it is made of
 * (the same selections and outputs; see below for the one fused step):
 *   MLA_LAYER_FULL, MLA_LAYER_REINDEX  the layer selects with its own indexer query over the
 *        shared indexer keys: for layer 0, mla_append_indexer_topk (the step's entry: main
 *        row, indexer key and layer 0's window entry, carried in the scan's launch where it
 *        can be); for a later layer, mla_indexer_topk (a Reindex layer scores only the pool
 *        when pool_blocks > 0); a Full layer with pool_blocks > 0 also writes its scores to
 *        pool_scores and publishes the pool (mla_indexer_pool) into pool_pos;
 *   MLA_LAYER_REUSE  the indices of the latest selecting layer;
 * then every layer's decode over the shared main cache with its own query and window:
 * mla_sparse_decode for layer 0, mla_append_sparse_decode (the layer's window entry
 * appended in the decode's call) for the others when W > 0. Selecting layers write their
 * indices to idx_a and idx_b in turn (the first to idx_a): with more than two selecting
 * layers, a buffer is overwritten by the selection two layers later. The bf16-score top-k
 * (mla_indexer_topk_bf16) when score_bf16 != 0.
 * One difference in how, not in what: for a capacity of 4096 rows or more and a decode on
 * the MFMA path (fmt E4M3_S128, E2M1_S16 or BF16 at 512 value channels), a selecting layer
 * (other than a Reindex layer scoring the pool) runs the many-workgroup selection and its
 * final step runs inside that layer's decode instead of as its own kernel (a Full layer that
 * publishes the pool then does so after its decode): the decode takes its rows from
 * the per-workgroup lists of the selection's first kernel and writes the index set to
 * idx_a or idx_b itself. The set is the one the separate calls select (an unordered set,
 * -1 in the same trailing slots); the order of its entries, and with it the decode's
 * summation order, may differ.
 *
 * One call instead of one per layer and kernel, for callers whose host loop would
 * otherwise set the pace: the launches are enqueued back to back from C.
 *
 *  layers        host array of n_layers descriptors (below); layer 0 must select
 *  new_main, new_idx, slots, n_new   the step's entry as for mla_append_indexer_topk
 *                (new_main NULL: the main row was appended by other means)
 *  main_cache, idx_cache, strides, capacity, n_visible, B, H, H_I, k, d_v   shared by the layers,
 *                as for the calls above
 *  win_pos, win_len, W, win_fmt   the layers' windows (W = 0: none); Dw = dim + rope
 *  pool_blocks, pool_block, pool_scores (fp32 [B, capacity]), pool_pos (int32
 *                [B, pool_blocks * pool_block])   the candidate pool, or pool_blocks = 0
 *  idx_a, idx_b  int32 [B, k] each
 *  topk_workspace   at least mla_indexer_topk_workspace (and mla_indexer_pool_workspace with
 *                a pool) bytes, under their zeroing contract; decode_workspace at least
 *                mla_sparse_decode_workspace(main_row, d_v, B, H, k, W, win_fmt) bytes
 * Errors: those of the calls above; and, before any launch, MLA_ERR_INVALID_ARG for an
 * unknown mode, a leading Reuse layer, a missing or misaligned per-layer pointer (q, out:
 * 16 bytes; q_idx 16, w 4 for selecting layers; win_ring 16 (MXFP8: 2), new_win 16 when
 * W > 0), missing index buffers or pool arrays, and MLA_ERR_WORKSPACE for a short workspace.
 */
enum { MLA_LAYER_FULL = 0, MLA_LAYER_REINDEX = 1, MLA_LAYER_REUSE = 2 };
typedef struct {
    int32_t mode;            /* MLA_LAYER_FULL, MLA_LAYER_REINDEX or MLA_LAYER_REUSE */
    const void* q;           /* [B, H, dim + rope] bf16: the layer's absorbed query */
    const void* q_idx;       /* [B, H_I, d_I] bf16: selecting layers (NULL for Reuse) */
    const float* w;          /* [B, H_I] indexer head weights: selecting layers */
    float* out;              /* [B, H, d_v] */
    float* lse;              /* [B, H] */
    void* win_ring;          /* the layer's window ring (bf16 or MXFP8 bytes), when W > 0 */
    const float* new_win;    /* [B, dim + rope] the step's window entry of the layer, when W > 0 */
} mla_group_layer_t;

mla_status_t mla_csa2_group_step(mla_row_t main_row, mla_row_t idx_row, int32_t d_v, int32_t n_layers,
                                 const mla_group_layer_t* layers, const float* new_main, const float* new_idx,
                                 const int32_t* slots, int32_t n_new, void* main_cache, int64_t main_seq_stride,
                                 void* idx_cache, int64_t idx_seq_stride, int64_t capacity,
                                 const int32_t* n_visible, int32_t B, int32_t H, int32_t H_I, int32_t k,
                                 float score_scale, float softmax_scale, const int32_t* win_pos,
                                 const int32_t* win_len, int32_t W, int32_t win_fmt, int32_t score_bf16,
                                 int32_t pool_blocks, int32_t pool_block, float* pool_scores, int32_t* pool_pos,
                                 int32_t* idx_a, int32_t* idx_b, void* topk_workspace, size_t topk_workspace_bytes,
                                 void* decode_workspace, size_t decode_workspace_bytes, void* stream);

/*
 * mla_sparse_decode_noalloc -- mla_sparse_decode with the library's own scratch.
 *
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation,
 * arguments and errors as mla_sparse_decode, without the workspace arguments.
 * The split partials (and an MXFP8 window's bf16 copy) go to a static array of
 * MLA_NOALLOC_SCRATCH_BYTES in device memory, one per GPU, held until the
 * process ends; the call allocates and frees nothing. Its device address is
 * looked up on the first call on each device, with that device current; the
 * stream must belong to the current device. Shapes whose workspace
 * (mla_sparse_decode_workspace) exceeds the array are rejected with
 * MLA_ERR_WORKSPACE. Every call on a GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams, or host threads without
 * ordering) race and give wrong results; order them on one stream.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (32u << 20)
mla_status_t mla_sparse_decode_noalloc(mla_row_t main_row, int32_t d_v, const void* q,
                                       const void* main_cache, int64_t main_seq_stride, int64_t capacity,
                                       const int32_t* idx, int32_t k,
                                       const void* win_ring, const int32_t* win_len, int32_t W,
                                       int32_t win_fmt, float softmax_scale,
                                       const mla_decode_epilogue_t* epilogue, int32_t B, int32_t H,
                                       float* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
