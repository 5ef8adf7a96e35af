// decode.hip -- absorbed-MLA sparse decode: shared-KV MQA over the selected
// latent entries plus the window, softmax, logsumexp output.
//
// For each (b, h), over U = {selected rows} + {window slots}:
//   z_u = scale * q[b,h,:] . K_u,  lse = logsumexp z,  out = sum_u e^(z_u - lse) K_u[:d_v]
// ([P1] "DeepSeek's Attention and KV Cache - From MLA to CSA2", "DeepSeek-V2",
// "Why RoPE breaks the trick" and "Check it in numpy"; [P2] "From MLA to DSA
// to HCA/CSA", Part 2 "What replaced MLA"; each selected latent is read once
// per head group of 16, [P1] "DeepSeek-V3.2", "The lightning indexer").
//
// MFMA path (H a multiple of 16 up to 128, d_v = 512, K width 576 = 512 + 64 or 512):
//   one workgroup of 8 waves per (b, split, group of 16 heads); a split is up
//   to 256 consecutive entries of idx[b] (E4M3 rows; 128 for bf16 and E2M1 rows
//   and for the window ring). Work items are laid out so that the head groups
//   of one split run on the same XCD and share its L2. The split's rows are
//   gathered into LDS at once (LDS DMA for E4M3 and bf16 rows; E2M1 rows
//   widened exactly to bf16 through registers), then QK (bf16 MFMA, E4M3 codes
//   widened exactly, one accumulator per 128-channel block times the row's
//   fp32 scale), an exact softmax over the split, and PV with each wave owning
//   64 value channels (V^T through ds_read_b64_tr_b8 / _b16, P times the E4M3
//   row's block scale as a high and a low bf16 term) -- see decode_split_g.
//   The split's normalised output and logsumexp are written as a partial and
//   k_merge combines the partials by logsumexp.
// Generic path (any other shape): one workgroup per (b, h), fp32 on the vector
// ALUs, writes the final output directly.
#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace mla {

namespace {

constexpr int kDv = 512;
constexpr int kMergeThreads = kDv / 4;
constexpr int kGenericThreads = 256;
constexpr int kGenericMaxRows = 8192;
constexpr int kMergeFast = 16;             // splits the merge loads in one round

enum SrcKind { SRC_E4M3 = 0, SRC_FP4 = 1, SRC_BF16 = 2, SRC_MX8 = 3 };   // SRC_MX8: MXFP8 window entries

typedef int v2i_t __attribute__((ext_vector_type(2)));
typedef short v4s_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 ds_tr8(const uint8_t* p) {
    const v2i_t r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i_t*)(
        (__attribute__((address_space(3))) uint8_t*)(uintptr_t)lds_addr(p)));
    return u32x2{(uint32_t)r.x, (uint32_t)r.y};
}
__device__ __forceinline__ u32x2 ds_tr16(const uint8_t* p) {
    const v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s_t*)(
        (__attribute__((address_space(3))) uint8_t*)(uintptr_t)lds_addr(p)));
    return u32x2{(uint32_t)(uint16_t)r.x | ((uint32_t)(uint16_t)r.y << 16),
                 (uint32_t)(uint16_t)r.z | ((uint32_t)(uint16_t)r.w << 16)};
}


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (round to nearest even, hardware convert), low half first
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
// 8 floats -> bf16 high parts and bf16 residuals (p = hi + lo to about 16 bits)
__device__ __forceinline__ void split_bf16x8(const float* p, u32x4& hi, u32x4& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h = pk_bf16(p[2 * i], p[2 * i + 1]);
        hi[i] = h;
        lo[i] = pk_bf16(p[2 * i] - u2f(h << 16), p[2 * i + 1] - u2f(h & 0xFFFF0000u));
    }
}


// 8 E4M3 codes -> 8 exact bf16 / fp16 values (two per u32)
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(u32x2 w) {
    const u32x2 a = e4m3x4_to_bf16(w.x), b = e4m3x4_to_bf16(w.y);
    return u32x4{a.x, a.y, b.x, b.y};
}

// ------------------------------------------------------------------------
// Gather-all split (8 waves, one head tile of 16 heads, up to R rows).
//
// A split's rows are gathered into LDS at once, as the value region: E4M3 rows
// as stored up to their RoPE part (512 codes | 4 fp32 block scales = 528 B,
// by LDS DMA, so the region is one contiguous image of 33 16-byte pieces per
// row); bf16 rows (and window entries) as their leading 512 channels (DMA, one
// row per load instruction, 1056-byte stride); E2M1 rows through registers,
// widened exactly to bf16 (E2M1 value times its E4M3 scale) in the same
// 1056-byte layout. RoPE channels (576-channel rows) are loaded per lane
// straight into the QK operand registers. The queries of the 16 heads sit in
// LDS. Then, with no per-chunk chain:
//   A  QK: wave w scores row tiles w, w + 8 (16 rows x 16 heads each) over the
//      whole K width (bf16 MFMA; E4M3 codes widened exactly, one accumulator per
//      128-channel block times the row's scale);
//   B  softmax over the split's rows, exact: the heads' maxima meet in LDS, P =
//      2^(z - max) goes to LDS (over the queries, no longer needed);
//   C  PV: wave w owns value channels 64 w .. 64 w + 63 for all 16 heads and
//      every row (V^T through the transposing LDS reads; P, times the E4M3 row's
//      block scale, as a high and a low bf16 term).
// The split's normalised output and logsumexp are its partial, merged by
// k_merge. One DMA wait and three barriers per workgroup; each CU gathers a
// split's rows once per head tile, at the rate its memory pipeline accepts them.
namespace gd {
constexpr int kQStride = 1168;                             // bytes per head of the staged queries (576 bf16 + 16 B)
template <int SRC>
struct VRow {
    static constexpr int kStride = SRC == SRC_E4M3 ? 528 : 1056;
    static constexpr int kRopeOff = SRC == SRC_E4M3 ? 528 : 1024;   // byte offset of a 576-channel row's RoPE part
};
template <int SRC, int R>
struct Lay {
    static constexpr int kVBytes = R * VRow<SRC>::kStride;
    static constexpr int kQ = kVBytes;                     // queries [16][kQStride], later P [16][R + 4] fp32
    static constexpr int kPStride = R + 4;
    static constexpr int kQBytes = (16 * kQStride > 16 * kPStride * 4) ? 16 * kQStride : 16 * kPStride * 4;
    static constexpr int kIdx = kQ + kQBytes;              // row indices [R]
    static constexpr int kRed = kIdx + R * 4;              // [2][8 waves][16 heads]: maxima, sums
    static constexpr int kBytes = kRed + 2 * 8 * 16 * 4;
};
template <int SRC_MAIN, int DQK>
constexpr int lds_bytes() {
    constexpr int m = Lay<SRC_MAIN, SRC_MAIN == SRC_E4M3 ? 256 : 128>::kBytes;
    constexpr int w = Lay<SRC_BF16, 128>::kBytes;
    return m > w ? m : w;
}
}  // namespace gd

// ---- finishing a many-workgroup selection inside the decode
// Slot o of sequence b's index set, placed as the selection's final places it: the rows
// above the threshold bin first, in the order of k_select's workgroups and of their lists;
// then the candidates of the threshold bin that the exact threshold takes (the composite
// key << 32 | ~position, so that equal scores go to the smaller position), in the same
// list order; -1 from min(n_visible, k) on ([P2] "CSA: two changes to HCA" for the -1
// slots). The workgroup of (b, split, head group) fills its split's slots first ..
// first + n - 1 into ridx (-1 for a position outside the cache); the splits that reach
// into the threshold bin run the radix over its candidates themselves (each head group
// of such a split, redundantly: the result is one function of the lists). scratch is
// the row buffers, free until the gather (candidates past its room go to one contiguous
// list in the workspace). Called by every thread of the workgroup.
namespace fs {
constexpr uint32_t kOffS = 0;                              // [kFusedSelectGroups + 1] selected offsets
constexpr uint32_t kOffC = 4160;                           // candidate offsets
constexpr uint32_t kHist = 8320;                           // [2][kMaxDigitBins] digit histograms
constexpr uint32_t kRes = 16512;                           // digit result
constexpr uint32_t kWsum = 16576;                          // [8 waves][2] scan totals
constexpr uint32_t kCand = 16640;                          // candidates
}  // namespace fs

__device__ void finish_selection(const DecodeArgs& a, uint8_t* scratch, uint32_t scratch_bytes, int32_t* ridx,
                                 int R, int b, bool zero_rest, int64_t first, int n) {
    static_assert(kFusedSelectGroups <= 2 * 512, "two workgroups' counts per thread");
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    uint32_t* offs_s = reinterpret_cast<uint32_t*>(scratch + fs::kOffS);
    uint32_t* offs_c = reinterpret_cast<uint32_t*>(scratch + fs::kOffC);
    uint32_t(*h)[kMaxDigitBins] = reinterpret_cast<uint32_t(*)[kMaxDigitBins]>(scratch + fs::kHist);
    uint32_t* res = reinterpret_cast<uint32_t*>(scratch + fs::kRes);
    uint32_t* wsum = reinterpret_cast<uint32_t*>(scratch + fs::kWsum);
    uint64_t* lc = reinterpret_cast<uint64_t*>(scratch + fs::kCand);
    const uint32_t cand_room = (scratch_bytes - fs::kCand) / 8;
    const int G = a.sel_groups;
    const int64_t cap = a.sel_capacity;
    const int64_t nvis = clamp_visible(a.sel_visible[b], cap);
    const uint32_t want = (uint32_t)(nvis < a.k ? nvis : a.k);
    uint32_t* hb = a.sel_hist + (int64_t)b * kHistWordsHost;
    const int32_t* sl = a.sel_lists + b * cap;
    const uint64_t* cl = a.cand_lists + b * cap;

    // the workgroups' counts (thread t: workgroups 2t, 2t + 1), exclusive prefix sums
    const uint32_t csum = (zero_rest && tid < 64) ? coarse_sum_of_lane(hb) : 0u;
    uint32_t cs[2], cc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = 2 * tid + i;
        const bool ok = j < G;
        const u32x2 c2 = *reinterpret_cast<const u32x2*>(a.sel_counts + ((int64_t)b * G + (ok ? j : 0)) * 2);
        cs[i] = ok ? c2.x : 0u;
        cc[i] = ok ? c2.y : 0u;
    }
    const uint32_t ts = cs[0] + cs[1], tc = cc[0] + cc[1];
    const uint32_t is = wave_incl_scan(ts), ic = wave_incl_scan(tc);
    if (lane == 63) {
        wsum[2 * wv] = is;
        wsum[2 * wv + 1] = ic;
    }
    lds_barrier();
    uint32_t bs = 0, bc = 0, nsel = 0, ncand = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t s_ = wsum[2 * i], c_ = wsum[2 * i + 1];
        if (i < wv) {
            bs += s_;
            bc += c_;
        }
        nsel += s_;
        ncand += c_;
    }
    const uint32_t es = bs + is - ts, ec = bc + ic - tc;
    if (2 * tid < G) {
        offs_s[2 * tid] = es;
        offs_c[2 * tid] = ec;
    }
    if (2 * tid + 1 < G) {
        offs_s[2 * tid + 1] = es + cs[0];
        offs_c[2 * tid + 1] = ec + cc[0];
    }
    lds_barrier();
    // the workgroup holding entry i of the concatenated lists: the last whose offset is <= i
    auto owner = [&](const uint32_t* offs, uint32_t i) {
        int lo = 0, hi = G - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (offs[mid] <= i) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    const int64_t o = first + tid;
    const uint32_t need = want > nsel ? want - nsel : 0u;
    const bool tail = need > 0 && first < (int64_t)want && first + n > (int64_t)nsel;
    const bool in_lds = ncand <= cand_room;
    // the split's selected slots and (in a split that reaches the threshold bin) the first
    // 2048 candidates, kCB consecutive ones per thread (one owner search, then a step to
    // the next list where one ends): every load issued before the first store
    constexpr int kCB = 4;                                 // candidates per thread per batch
    auto load_run = [&](uint32_t i0, uint64_t* v) {
        int j = i0 < ncand ? owner(offs_c, i0) : 0;
#pragma unroll
        for (int u = 0; u < kCB; ++u) {
            const uint32_t i = i0 + u;
            v[u] = 0ull;
            if (i < ncand) {
                while (j + 1 < G && offs_c[j + 1] <= i) ++j;
                v[u] = cl[(int64_t)j * kSelRowsHost + (i - offs_c[j])];
            }
        }
    };
    int32_t r = -1;
    if (tid < n && o < (int64_t)nsel) {
        const int j = owner(offs_s, (uint32_t)o);
        r = sl[(int64_t)j * kSelRowsHost + ((uint32_t)o - offs_s[j])];
    }
    uint64_t cv0[kCB];
    if (tail && in_lds) load_run(kCB * tid, cv0);
    if (tid < R) ridx[tid] = (r >= 0 && r < a.capacity) ? r : -1;
    if (tail) {
        if (in_lds) {
#pragma unroll
            for (int u = 0; u < kCB; ++u) {
                const uint32_t i = kCB * tid + u;
                if (i < ncand) lc[i] = cv0[u];
            }
            for (uint32_t b0 = kCB * 512; b0 < ncand; b0 += kCB * 512) {
                uint64_t v[kCB];
                load_run(b0 + kCB * tid, v);
#pragma unroll
                for (int u = 0; u < kCB; ++u) {
                    const uint32_t i = b0 + kCB * tid + u;
                    if (i < ncand) lc[i] = v[u];
                }
            }
        } else {
            // past the room: one contiguous copy in the workspace, written alike by every workgroup
            // that finishes this sequence (the same bytes), read back by this one after its fence
            uint64_t* cf = a.cand_flat + b * cap;
            for (uint32_t b0 = 0; b0 < ncand; b0 += kCB * 512) {
                uint64_t v[kCB];
                load_run(b0 + kCB * tid, v);
#pragma unroll
                for (int u = 0; u < kCB; ++u) {
                    const uint32_t i = b0 + kCB * tid + u;
                    if (i < ncand) cf[i] = v[u];
                }
            }
            __threadfence_block();
        }
        for (int i = tid; i < 2 * kMaxDigitBins; i += 512) h[0][i] = 0u;
        __syncthreads();
        // the radix and the ranking, over the candidates in LDS or (past its room) in the lists
        auto finish = [&](auto cv) {
            // the radix over the candidates' composites, most significant digit first: two
            // 10-bit digits fix the threshold score (the bin fixed its top 12 bits; the second
            // only when the first leaves more candidates than are still needed), and digits of
            // the inverted position follow when more candidates share that score than are
            // still needed; `prefix` ends as the need-th largest composite
            const bool radix = need < ncand;
            uint64_t mask = 0xFFFull << 52, prefix = radix ? (cv(0) & mask) : 0ull;
            uint32_t rem = need;
            int par = 0;
            auto pass = [&](int shift, int bits) {
                const int nb = 1 << bits;
                uint32_t* hc = h[par];
                for (uint32_t i = tid; i < ncand; i += 512) {
                    const uint64_t v = cv(i);
                    if ((v & mask) == prefix) atomicAdd(&hc[(v >> shift) & (uint64_t)(nb - 1)], 1u);
                }
                lds_barrier();
                if (tid < 64) {
                    const DigitResult d = wave_find_digit(hc, nb, rem);
                    if (lane == 0) {
                        res[0] = (uint32_t)d.digit;
                        res[1] = d.above;
                        res[2] = d.count;
                    }
                } else {
                    for (int i = tid - 64; i < kMaxDigitBins; i += 512 - 64) h[par ^ 1][i] = 0u;
                }
                lds_barrier();
                prefix |= (uint64_t)res[0] << shift;
                mask |= (uint64_t)(nb - 1) << shift;
                rem -= res[1];
                par ^= 1;
                return res[2];
            };
            if (radix) {
                const uint32_t c1 = pass(42, 10);
                if (rem < c1) {                            // (every candidate of the digit needed: done)
                    const uint32_t eq = pass(32, 10);
                    if (rem < eq) {
                        // ties at the threshold score: the inverted position's digits. Positions
                        // lie below the capacity, so its bits from pb up are ones in every
                        // candidate; the digits cover bits pb - 1 .. 0 from the top, 10 at a time
                        // (the last of 8 or 10 bits, reaching below 0 into bits already fixed)
                        const int pb = 32 - __builtin_clz((uint32_t)(cap > 1 ? cap - 1 : 1));
                        const uint64_t ones = pb < 32 ? (uint64_t)(0xFFFFFFFFu >> pb << pb) : 0ull;
                        prefix |= ones;
                        mask |= ones;
                        for (int hi = pb; hi > 0;) {
                            const int bits = hi >= 10 ? 10 : (hi > 8 ? 10 : 8);
                            const int lo = hi - bits > 0 ? hi - bits : 0;
                            pass(lo, bits);
                            hi = lo;
                        }
                    }
                }
            }
            // the taken candidates (every one at or above `prefix`: exactly `need`), ranked in list
            // order; rank q fills slot nsel + q, and this split keeps the ranks of its own slots
            const uint32_t q_lo = (uint32_t)((first > (int64_t)nsel ? first : (int64_t)nsel) - nsel);
            const uint32_t q_hi = (uint32_t)((first + n < (int64_t)want ? first + n : (int64_t)want) - nsel);
            uint32_t base = 0;
            int it = 0;
            for (uint32_t i0 = 0; i0 < ncand && base < q_hi; i0 += 512, ++it) {
                const uint32_t i = i0 + tid;
                const uint64_t v = i < ncand ? cv(i) : 0ull;
                const bool take = i < ncand && (!radix || v >= prefix);
                const uint64_t m = __ballot(take);
                uint32_t* ws2 = wsum + 8 * (it & 1);           // two sets: one barrier per round
                if (lane == 0) ws2[wv] = (uint32_t)__popcll(m);
                lds_barrier();
                uint32_t before = 0, tot = 0;
    #pragma unroll
                for (int w2 = 0; w2 < 8; ++w2) {
                    const uint32_t c_ = ws2[w2];
                    if (w2 < wv) before += c_;
                    tot += c_;
                }
                if (take) {
                    const uint32_t q = base + before + lanes_below(m);
                    if (q >= q_lo && q < q_hi) {
                        const int32_t pos = (int32_t)~(uint32_t)(v & 0xFFFFFFFFull);
                        ridx[(int64_t)nsel + q - first] = (pos >= 0 && pos < a.capacity) ? pos : -1;
                    }
                }
                base += tot;
            }
        };
        if (in_lds) finish([&](uint32_t i) { return lc[i]; });
        else finish([&](uint32_t i) { return a.cand_flat[b * cap + i]; });
    }
    if (zero_rest) zero_hist_rest(hb, (uint32_t)a.k, csum);
}

template <int SRC, int DQK, int R>
__device__ __forceinline__ void decode_split_g(const DecodeArgs& a, uint8_t* smem, int b, int split, int S, int hg,
                                               bool is_win, int64_t first, int n, int span, float* o_part,
                                               float* lse_part) {
    using L = gd::Lay<SRC, R>;
    constexpr int VS = gd::VRow<SRC>::kStride;
    constexpr int NT = (R / 16 + 7) / 8;                   // row tiles per wave (waves w < R / 16 have them)
    constexpr bool kRope = DQK == 576;
    constexpr int NMAIN = 16;                              // k-steps of 32 channels in the value region
    // E4M3 splits of 256 rows are gathered in two halves (rows 0 .. 127, then 128 .. 255), and
    // the first row tile of every wave (in the first half) is contracted while the second lands
    constexpr int NPART = (SRC == SRC_E4M3 && NT == 2 && R == 256) ? 2 : 1;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = lane & 15, g = lane >> 4;
    uint8_t* V = smem;
    uint8_t* Q = smem + L::kQ;
    float* P = reinterpret_cast<float*>(smem + L::kQ);
    int32_t* ridx = reinterpret_cast<int32_t*>(smem + L::kIdx);
    float* red = reinterpret_cast<float*>(smem + L::kRed);
    constexpr float kLog2e = 1.4426950408889634f;
    const float zscale = a.scale * kLog2e;
    static_assert(SRC != SRC_MX8 || DQK == 512, "MXFP8 window entries of 512 channels");
    constexpr uint32_t kMx8Bytes = DQK + DQK / 32;        // an MXFP8 entry: codes, then one E8M0 byte per 32
    const uint8_t* row_base = SRC == SRC_MX8 ? a.win8 + (int64_t)b * a.W * kMx8Bytes
                              : is_win       ? reinterpret_cast<const uint8_t*>(a.win + (int64_t)b * a.W * DQK)
                                             : a.cache + b * a.stride;
    const uint32_t row_bytes = SRC == SRC_MX8 ? kMx8Bytes : is_win ? 2 * DQK : (uint32_t)a.row_bytes;

    // the step's window entry, when its ring slot lies in this window split's span of slots:
    // row u_new of the split is staged from it (attended when u_new < n) and, by head group
    // 0, written into the ring, instead of read
    int u_new = -1;
    int64_t s_new = 0;
    f32x4 nw0 = f32x4{0.f, 0.f, 0.f, 0.f}, nw1 = nw0;     // bf16 windows: this lane's 8 channels of the entry
    if constexpr ((SRC == SRC_BF16 || SRC == SRC_MX8) && DQK == 512) {
        if (is_win && a.new_win) {
            const int64_t pos = a.win_pos[b];
            s_new = pos >= 0 ? pos % a.W : -1;
            if (s_new >= first && s_new < first + span) u_new = (int)(s_new - first);
        }
    }

    // ---- row indices (-1: no row) and the 16 heads' queries (their loads issued first)
    {
        constexpr int kPer = DQK / 8;                      // 16-byte pieces per head
        constexpr int kIt = (16 * kPer + 511) / 512;
        const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.H + 16 * hg) * DQK;
        u32x4 qv[kIt];
#pragma unroll
        for (int i = 0; i < kIt; ++i) {                    // every load issued before the first store
            const int it = tid + 512 * i, h = it / kPer, pc = it - h * kPer;
            if (it < 16 * kPer) qv[i] = *reinterpret_cast<const u32x4*>(qsrc + (int64_t)h * DQK + 8 * pc);
        }
        if (!is_win && a.sel_counts) {                     // the rows of a selection this decode finishes
            finish_selection(a, V, (uint32_t)L::kVBytes, ridx, R, b, split == 0 && hg == 0, first, n);
        } else if (tid < R) {
            int32_t r = -1;
            if (tid < n) {
                if (is_win) r = (int32_t)(first + tid);
                else {
                    const int32_t s = a.idx[(int64_t)b * a.k + first + tid];
                    if (s >= 0 && s < a.capacity) r = s;
                }
            }
            ridx[tid] = r;
        }
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int it = tid + 512 * i, h = it / kPer, pc = it - h * kPer;
            if (it < 16 * kPer) *reinterpret_cast<u32x4*>(Q + h * gd::kQStride + 16 * pc) = qv[i];
        }
    }
    __syncthreads();
    if (!is_win && a.sel_counts && hg == 0 && tid < n)    // the finished index set, once per split
        a.idx_out[(int64_t)b * a.k + first + tid] = ridx[tid];
    // B operands of the contraction (lane (head j, g): channels 32 s + 8 g .. of head j), read
    // from LDS now so that the reads overlap the gather
    constexpr int NQ = DQK / 32;                           // k-steps over the K width
    u32x4 qv[NQ];
    {
        const uint8_t* qh = Q + j * gd::kQStride + 16 * g;
#pragma unroll
        for (int st = 0; st < NQ; ++st) qv[st] = *reinterpret_cast<const u32x4*>(qh + 64 * st);
    }

    // ---- gather the value region; slots without a row load a stand-in and are zeroed once landed
    const uint32_t v_m0 = __builtin_amdgcn_readfirstlane(lds_addr(V));
    uint32_t zmask = 0;
    if constexpr (SRC == SRC_E4M3) {
        constexpr int NI = R * 33 / 64;                   // load instructions: 33 pieces per row, 64 per load
        constexpr int NH = NI / NPART;                    // per part (a half: 66 loads = 128 rows)
        constexpr int PW = (NH + 7) / 8;
        static_assert(NH * NPART == NI && (NPART == 1 || (NH * 64) % 33 == 0), "parts of whole rows");
        // the head groups of a split (one XCD) gather the same rows: each starts at a different
        // eighth of each part, so that a row's first requests come from different head groups
        // and the L2 merges the others into them; every load is issued at once (waiting for the
        // group's own eighth before requesting the rest cost a memory round trip)
        const int rot = ((hg & 7) * (NH / 8)) & ~7;
#pragma unroll
        for (int part = 0; part < NPART; ++part)
#pragma unroll
        for (int i = 0; i < PW; ++i) {
            int I = w + 8 * i;
            if (I < NH) {
                I = part * NH + (I + rot) % NH;
                const int P16 = 64 * I + lane;
                const int u = P16 / 33, pc = P16 - 33 * u;
                const int32_t r = ridx[u];
                zmask |= r < 0 ? (1u << (part * PW + i)) : 0u;
                const uint8_t* src = r >= 0 ? row_base + (uint64_t)(uint32_t)r * row_bytes + 16 * pc
                                            : reinterpret_cast<const uint8_t*>(a.q);
                dma16(src, __builtin_amdgcn_readfirstlane(v_m0 + 1024u * (uint32_t)I));
            }
        }
    } else if constexpr (SRC == SRC_BF16) {
        constexpr int PW = R / 8;                          // one row per load instruction
        const int rot = (hg & 7) * (R / 8);                // (a multiple of 8: a wave keeps its rows)
        if constexpr (DQK == 512) {                        // the wave whose rows hold u_new loads the entry now
            if (u_new >= 0 && (u_new & 7) == w) {
                const float* src = a.new_win + (int64_t)b * DQK + 8 * lane;
                nw0 = *reinterpret_cast<const f32x4*>(src);
                nw1 = *reinterpret_cast<const f32x4*>(src + 4);
            }
        }
#pragma unroll 4
        for (int i = 0; i < PW; ++i) {
            if (i == (PW + 7) / 8) wait_vmcnt<0>();       // the group's own eighth first, landed before the rest
            const int u = (w + 8 * i + rot) % R;
            const int32_t r = u == u_new ? -1 : ridx[u];   // (the new entry's row: a stand-in, then overwritten)
            zmask |= r < 0 ? (1u << i) : 0u;
            const uint8_t* src = r >= 0 ? row_base + (uint64_t)(uint32_t)r * row_bytes + 16 * lane
                                        : reinterpret_cast<const uint8_t*>(a.q);
            dma16(src, __builtin_amdgcn_readfirstlane(v_m0 + (uint32_t)(VS * u)));
        }
    } else if constexpr (SRC == SRC_MX8) {                 // MXFP8 entries: 16 blocks of 32 channels per entry
        // (one E8M0 scale per block: the converter applies the power of two given as an
        // fp32 scale, whose exponent field is the E8M0 code; E4M3 times 2^k is exact in
        // bf16 down to bf16's subnormals, as with the entry widened on its own)
        constexpr int kPer = R * 16 / 512;
        u32x4 c0[kPer], c1[kPer];
        uint32_t scb[kPer];
        // the wave that stages the new entry's row (16 threads of it) quantises the whole
        // entry afterwards, 8 channels per lane, and writes it over that row: load them now
        const int w_new = u_new >= 0 ? ((16 * u_new) & 511) >> 6 : -1;
        if (w == w_new) {
            const float* src = a.new_win + (int64_t)b * DQK + 8 * lane;
            nw0 = *reinterpret_cast<const f32x4*>(src);
            nw1 = *reinterpret_cast<const f32x4*>(src + 4);
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int item = tid + 512 * i, u = item >> 4, pc = item & 15;
            const int32_t r = ridx[u];
            const uint8_t* rp = row_base + (uint64_t)(uint32_t)(r < 0 ? 0 : r) * row_bytes;
            c0[i] = r >= 0 ? *reinterpret_cast<const u32x4*>(rp + 32 * pc) : u32x4{0u, 0u, 0u, 0u};
            c1[i] = r >= 0 ? *reinterpret_cast<const u32x4*>(rp + 32 * pc + 16) : u32x4{0u, 0u, 0u, 0u};
            scb[i] = r >= 0 ? (uint32_t)rp[DQK + pc] : 127u;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int item = tid + 512 * i, u = item >> 4, pc = item & 15;
            u32x4* d = reinterpret_cast<u32x4*>(V + u * VS + 64 * pc);
            const float sc = u2f(scb[i] << 23);            // exponent field = the E8M0 code
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const u32x4 c = h2 ? c1[i] : c0[i];
#pragma unroll
                for (int q2 = 0; q2 < 2; ++q2) {
                    const uint32_t w0 = c[2 * q2], w1 = c[2 * q2 + 1];
                    d[2 * h2 + q2] = u32x4{
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, sc, true)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, false)),
                        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, sc, true))};
                }
            }
        }
        if (w == w_new) {                                  // the entry, quantised as the append quantises it
            const float x[8] = {nw0[0], nw0[1], nw0[2], nw0[3], nw1[0], nw1[1], nw1[2], nw1[3]};
            uint32_t m = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = max(m, f2u(fabsf(x[e])));
            m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));           // the 4 lanes of a 32-channel block
            m = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
            const uint32_t code = mx8_code(m);
            const int sh = 127 - (int)code;
            uint32_t wd[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                wd[e >> 2] |= (m == 0u ? 0u : e4m3_encode(__builtin_ldexpf(x[e], sh))) << (8 * (e & 3));
            const float sc = u2f(code << 23);
            *reinterpret_cast<u32x4*>(V + u_new * VS + 16 * lane) = u32x4{
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[0], sc, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[0], sc, true)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[1], sc, false)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd[1], sc, true))};
            if (hg == 0) {
                uint8_t* ent = const_cast<uint8_t*>(a.win8) + ((int64_t)b * a.W + s_new) * kMx8Bytes;
                *reinterpret_cast<u32x2*>(ent + 8 * lane) = u32x2{wd[0], wd[1]};
                if ((lane & 3) == 0) ent[DQK + (lane >> 2)] = (uint8_t)code;
            }
        }
    } else {                                               // E2M1 rows: 16 pieces of 32 channels per row
        constexpr int kPer = R * 16 / 512;
        u32x4 nib[kPer];
        uint32_t scb[kPer];
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int item = tid + 512 * i, u = item >> 4, pc = item & 15;
            const int32_t r = ridx[u];
            const uint8_t* rp = row_base + (uint64_t)(uint32_t)(r < 0 ? 0 : r) * row_bytes;
            nib[i] = r >= 0 ? *reinterpret_cast<const u32x4*>(rp + 16 * pc) : u32x4{0u, 0u, 0u, 0u};
            scb[i] = r >= 0 ? *reinterpret_cast<const uint16_t*>(rp + 256 + 2 * pc) : 0u;
        }
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int item = tid + 512 * i, u = item >> 4, pc = item & 15;
            u32x4* d = reinterpret_cast<u32x4*>(V + u * VS + 64 * pc);
            const float s0 = e4m3_to_f32(scb[i] & 0xFFu), s1 = e4m3_to_f32((scb[i] >> 8) & 0xFFu);
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float sc = q4 < 2 ? s0 : s1;
                const uint32_t wv = nib[i][q4];
                const f32x2 v0 = e2m1x2_to_f32<0>(wv), v1 = e2m1x2_to_f32<1>(wv);
                const f32x2 v2 = e2m1x2_to_f32<2>(wv), v3 = e2m1x2_to_f32<3>(wv);
                d[q4] = u32x4{pack_bf16_trunc(v0.x * sc, v0.y * sc), pack_bf16_trunc(v1.x * sc, v1.y * sc),
                              pack_bf16_trunc(v2.x * sc, v2.y * sc), pack_bf16_trunc(v3.x * sc, v3.y * sc)};
            }
        }
    }
    // RoPE channels of the wave's row tiles, straight into QK operand registers (A layout:
    // lane (row j, k-group g) holds channels 512 + 32 s + 8 g .. + 7 of its row)
    u32x4 rope[NT][2];
    if constexpr (kRope) {
#pragma unroll
        for (int m = 0; m < NT; ++m) {
            const int tt = w + 8 * m;
            const int32_t r = (16 * tt < R) ? ridx[16 * tt + j] : -1;
            const uint8_t* rp = row_base + (uint64_t)(uint32_t)(r < 0 ? 0 : r) * row_bytes + gd::VRow<SRC>::kRopeOff;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                rope[m][s2] = r >= 0 ? *reinterpret_cast<const u32x4*>(rp + 2 * (32 * s2 + 8 * g))
                                     : u32x4{0u, 0u, 0u, 0u};
        }
    }
    // ---- A: scores of the wave's row tiles; lane (head j, g) ends with rows 4 g .. 4 g + 3 of each tile.
    // The value-region part of tile m (main), then its RoPE part (rope), in this order for every tile
    f32x4 acc[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto live = [&](int m) { return 16 * (w + 8 * m) < n; };   // (wave-uniform) a tile with a row of the split
    auto qk_main = [&](int m) {
        const int tt = w + 8 * m;
        const uint8_t* krow = V + (16 * tt + j) * VS;
        if constexpr (SRC == SRC_E4M3) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                f32x4 t4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s4 = 0; s4 < 4; ++s4) {
                    const int st = 4 * blk + s4;
                    const u32x2 codes = *reinterpret_cast<const u32x2*>(krow + 32 * st + 8 * g);
                    t4 = mfma_bf16(e4m3x8_to_bf16(codes), qv[st], t4);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    acc[m][r] += t4[r] * *reinterpret_cast<const float*>(V + (16 * tt + 4 * g + r) * VS + 512 + 4 * blk);
            }
        } else {
#pragma unroll
            for (int st = 0; st < NMAIN; ++st)
                acc[m] = mfma_bf16(*reinterpret_cast<const u32x4*>(krow + 2 * (32 * st + 8 * g)), qv[st], acc[m]);
        }
    };
    if constexpr (NPART == 2) {
        // this wave's first half has landed once at most the second half's loads are
        // outstanding (wave 7 issues the fewest of them); the whole first half after the barrier
        constexpr int kSecond = (R * 33 / 64 / 2 - 1 - 7) / 8 + 1;
        wait_vmcnt<kSecond>();
        lds_barrier();
        if (live(0)) qk_main(0);
    }
    wait_vmcnt<0>();
    if constexpr (SRC == SRC_E4M3) {
        // slots without a row: zeroed for PV (their scores are masked below, so the
        // first half's contraction may have read them before or after)
        constexpr int NI = R * 33 / 64;
        constexpr int NH = NI / NPART;
        constexpr int PW = (NH + 7) / 8;
        const int rot = ((hg & 7) * (NH / 8)) & ~7;
        if (__builtin_amdgcn_ballot_w64(zmask != 0u)) {
#pragma unroll
            for (int part = 0; part < NPART; ++part)
#pragma unroll
                for (int i = 0; i < PW; ++i)
                    if ((zmask >> (part * PW + i)) & 1u)
                        *reinterpret_cast<u32x4*>(V + 16 * (64 * (part * NH + (w + 8 * i + rot) % NH) + lane)) =
                            u32x4{0u, 0u, 0u, 0u};
        }
    } else if constexpr (SRC == SRC_BF16) {
        const int rot = (hg & 7) * (R / 8);
        if (__builtin_amdgcn_ballot_w64(zmask != 0u)) {
            for (int i = 0; i < R / 8; ++i)
                if ((zmask >> i) & 1u)
                    *reinterpret_cast<u32x4*>(V + VS * ((w + 8 * i + rot) % R) + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (DQK == 512) {
            if (u_new >= 0 && (u_new & 7) == w) {          // the step's entry, rounded to bf16 as the append does
                const u32x4 v = u32x4{bf16_rne(nw0[0]) | (bf16_rne(nw0[1]) << 16), bf16_rne(nw0[2]) | (bf16_rne(nw0[3]) << 16),
                                      bf16_rne(nw1[0]) | (bf16_rne(nw1[1]) << 16), bf16_rne(nw1[2]) | (bf16_rne(nw1[3]) << 16)};
                *reinterpret_cast<u32x4*>(V + VS * u_new + 16 * lane) = v;
                if (hg == 0)
                    *reinterpret_cast<u32x4*>(const_cast<uint16_t*>(a.win) + ((int64_t)b * a.W + s_new) * DQK + 8 * lane) = v;
            }
        }
    }
    __syncthreads();

    float z[NT][4];
#pragma unroll
    for (int m = 0; m < NT; ++m) {
        const int tt = w + 8 * m;
        if (live(m)) {
            if (NPART == 1 || m > 0) qk_main(m);
            if constexpr (kRope) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2)
                    acc[m] = mfma_bf16(rope[m][s2], qv[NMAIN + s2], acc[m]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * tt + 4 * g + r;
            z[m][r] = (live(m) && ridx[row] >= 0) ? acc[m][r] * zscale : -__builtin_inff();
        }
    }

    // ---- B: exact softmax over the split's rows (base 2)
    float mloc = -__builtin_inff();
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) mloc = fmaxf(mloc, z[m][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    if (g == 0) red[16 * w + j] = mloc;
    __syncthreads();                                       // maxima in; every wave is past its query reads
    float M = red[j];
#pragma unroll
    for (int ww = 1; ww < 8; ++ww) M = fmaxf(M, red[16 * ww + j]);
    float sloc = 0.0f;
#pragma unroll
    for (int m = 0; m < NT; ++m) {
        const int tt = w + 8 * m;
        f32x4 pv4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pv4[r] = (z[m][r] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(z[m][r] - M);
            sloc += pv4[r];
        }
        if (16 * tt < R) *reinterpret_cast<f32x4*>(P + j * L::kPStride + 16 * tt + 4 * g) = pv4;
    }
    sloc += __shfl_xor(sloc, 16, 64);
    sloc += __shfl_xor(sloc, 32, 64);
    if (g == 0) red[128 + 16 * w + j] = sloc;
    __syncthreads();                                       // P and the sums in

    // ---- C: PV over every row for value channels 64 w .. 64 w + 63
    f32x4 o[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int blk = w >> 1;                                // the E4M3 block of the wave's channels
    for (int st = 0; st < R / 32; ++st) {
        if (32 * st >= n) break;
        const float* pr = P + j * L::kPStride + 32 * st + 8 * g;
        const f32x4 p0 = *reinterpret_cast<const f32x4*>(pr), p1 = *reinterpret_cast<const f32x4*>(pr + 4);
        float p[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
        if constexpr (SRC == SRC_E4M3) {
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] *= *reinterpret_cast<const float*>(V + (32 * st + 8 * g + e) * VS + 512 + 4 * blk);
        }
        u32x4 pa, pb;
        split_bf16x8(p, pa, pb);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int c0 = 64 * w + 16 * mt;
            u32x4 av;
            if constexpr (SRC == SRC_E4M3) {
                av = e4m3x8_to_bf16(ds_tr8(V + (32 * st + 8 * g + (j >> 1)) * VS + c0 + 8 * (j & 1)));
            } else {
                const uint8_t* vp = V + (32 * st + 8 * g + (j >> 2)) * VS + 2 * (c0 + 4 * (j & 3));
                const u32x2 r0 = ds_tr16(vp), r1 = ds_tr16(vp + 4 * VS);
                av = u32x4{r0.x, r0.y, r1.x, r1.y};
            }
            o[mt] = mfma_bf16(av, pa, o[mt]);
            o[mt] = mfma_bf16(av, pb, o[mt]);
        }
    }

    // ---- the split's partial: normalised output (channels 64 w ..) and logsumexp (natural log)
    float l = red[128 + j];
#pragma unroll
    for (int ww = 1; ww < 8; ++ww) l += red[128 + 16 * ww + j];
    const int head = 16 * hg + j;
    const int64_t prow = ((int64_t)b * S + split) * a.H + head;
    const float f = (l > 0.0f) ? __builtin_amdgcn_rcpf(l) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
        *reinterpret_cast<float4*>(o_part + prow * kDv + 64 * w + 16 * mt + 4 * g) =
            make_float4(o[mt][0] * f, o[mt][1] * f, o[mt][2] * f, o[mt][3] * f);
    if (w == 0 && g == 0)
        lse_part[prow] = (l > 0.0f) ? (M + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : -__builtin_inff();
}

// Split for bf16 rows (and bf16 window entries), two head tiles of 16 heads per
// workgroup: waves 0-3 serve heads 32 hp .. + 15, waves 4-7 heads 32 hp + 16 .. + 31,
// over the same staged rows, so each row crosses into a CU once per 32 heads. A split
// of up to kMaxRows rows streams through two LDS buffers of kC rows: the next chunk's
// rows are gathered while the current one is contracted, and the softmax runs online
// over the chunks (running maximum per head; the output and the running sum rescaled
// when it grows), so one workgroup per CU covers as many rows as one round of the CUs
// needs and the split's partial is written once. The queries go from memory straight
// into each wave's operand registers. Per chunk: QK on the wave's row tile, the chunk's
// maximum per head tile, P for the chunk, PV with the wave owning 64 value channels of
// both head tiles (each V^T operand read from LDS once for the 32 heads). The pairs of a split (one XCD) take its chunks in rotated order, so
// that a chunk's rows come from HBM for one pair and from the L2 for the others.
namespace gd2 {
constexpr int kC = 64;                                     // rows per chunk
constexpr int kMaxRows = 512;                              // rows per split at most
constexpr int kVS = 1056;                                  // bytes per staged row (512 bf16 + 32)
constexpr int kBuf = kC * kVS;                             // one chunk's rows
constexpr int kPStride = kC + 4;                           // fp32 per head in P
constexpr int kP = 2 * kBuf;                               // P [32 heads][kPStride]
constexpr int kIdx = kP + 32 * kPStride * 4;               // row indices [kMaxRows]
constexpr int kRed = kIdx + kMaxRows * 4;                  // [2][8 waves][16 heads]
constexpr int kBytes = kRed + 2 * 8 * 16 * 4;
}  // namespace gd2

template <int DQK>
__device__ __forceinline__ void decode_split_pair(const DecodeArgs& a, uint8_t* smem, int b, int split, int S,
                                                  int hp, bool is_win, int64_t first, int n, float* o_part,
                                                  float* lse_part) {
    constexpr int C = gd2::kC, VS = gd2::kVS;
    constexpr bool kRope = DQK == 576;
    constexpr int NMAIN = 16, NQ = DQK / 32;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hs = w >> 2, wq = w & 3;                     // the wave's head tile in the pair, its row tile
    const int j = lane & 15, g = lane >> 4;
    uint8_t* V = smem;
    float* P = reinterpret_cast<float*>(smem + gd2::kP);
    int32_t* ridx = reinterpret_cast<int32_t*>(smem + gd2::kIdx);
    float* red = reinterpret_cast<float*>(smem + gd2::kRed);
    constexpr float kLog2e = 1.4426950408889634f;
    constexpr float kNegInf = -__builtin_inff();
    const float zscale = a.scale * kLog2e;
    const uint8_t* row_base = is_win ? reinterpret_cast<const uint8_t*>(a.win + (int64_t)b * a.W * DQK)
                                     : a.cache + b * a.stride;
    const uint32_t row_bytes = is_win ? 2 * DQK : (uint32_t)a.row_bytes;
    const int nch = (n + C - 1) / C;                       // n <= kMaxRows (the launcher's split)

    // the pair's 32 heads' queries (registers, then LDS in the second row buffer) and the
    // row indices (thread u: row u of the split; -1 past n, negative or out of range),
    // every load issued before the first store
    constexpr int kPer = DQK / 8;                          // 16-byte pieces per head
    constexpr int kIt = (32 * kPer + 511) / 512;
    static_assert(gd2::kBuf + 32 * gd::kQStride <= 2 * gd2::kBuf, "the staged queries fit the second buffer");
    static_assert(gd2::kMaxRows <= 512, "one row index per thread");
    uint8_t* Q = V + gd2::kBuf;
    {
        const uint16_t* qsrc = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.H + 32 * hp) * DQK;
        u32x4 qs[kIt];
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int it = tid + 512 * i, hh = it / kPer, pc = it - hh * kPer;
            if (it < 32 * kPer) qs[i] = *reinterpret_cast<const u32x4*>(qsrc + (int64_t)hh * DQK + 8 * pc);
        }
        if (!is_win && a.sel_counts) {                     // the rows of a selection this decode finishes
            finish_selection(a, V, 2 * gd2::kBuf, ridx, nch * C, b, split == 0 && hp == 0, first, n);
            lds_barrier();                                 // (the row buffers were its scratch)
        } else {
            int32_t r = -1;
            if (tid < n) {
                if (is_win) r = (int32_t)(first + tid);
                else {
                    const int32_t s = a.idx[(int64_t)b * a.k + first + tid];
                    if (s >= 0 && s < a.capacity) r = s;
                }
            }
            if (tid < nch * C) ridx[tid] = r;
        }
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int it = tid + 512 * i, hh = it / kPer, pc = it - hh * kPer;
            if (it < 32 * kPer) *reinterpret_cast<u32x4*>(Q + hh * gd::kQStride + 16 * pc) = qs[i];
        }
    }
    __syncthreads();                                       // the row indices and the queries
    if (!is_win && a.sel_counts && hp == 0 && tid < n)    // the finished index set, once per split
        a.idx_out[(int64_t)b * a.k + first + tid] = ridx[tid];

    const uint32_t v_m0 = __builtin_amdgcn_readfirstlane(lds_addr(V));
    const int rot = nch > 0 ? hp % nch : 0;
    auto chunk_of = [&](int c) { const int cc = c + rot; return cc >= nch ? cc - nch : cc; };
    // gather chunk c into buffer c & 1: one row per load instruction (wave w: rows w + 8 i),
    // rows with no entry loaded from the queries (any readable bytes) and zeroed once landed;
    // the RoPE part of the wave's row tile straight into registers
    u32x4 rope_c[2], rope_n[2];
    uint32_t zm_c = 0, zm_n = 0;
    auto issue = [&](int c) {
        const int base = C * chunk_of(c);
        const uint32_t m0 = v_m0 + (uint32_t)((c & 1) * gd2::kBuf);
        uint32_t zm = 0;
        const int32_t rv = ridx[base + w + 8 * (lane & 7)];  // lane i < 8: the entry of row w + 8 i
#pragma unroll
        for (int i = 0; i < C / 8; ++i) {
            const int u = w + 8 * i;
            const int32_t r = __builtin_amdgcn_readlane(rv, i);
            zm |= r < 0 ? (1u << i) : 0u;
            const uint8_t* src = r >= 0 ? row_base + (uint64_t)(uint32_t)r * row_bytes + 16 * lane
                                        : reinterpret_cast<const uint8_t*>(a.q);
            dma16(src, __builtin_amdgcn_readfirstlane(m0 + (uint32_t)(VS * u)));
        }
        zm_n = zm;
        if constexpr (kRope) {
            const int32_t r = ridx[base + 16 * wq + j];
            const uint8_t* rp = row_base + (uint64_t)(uint32_t)(r < 0 ? 0 : r) * row_bytes + 1024;
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
                rope_n[s2] = r >= 0 ? *reinterpret_cast<const u32x4*>(rp + 2 * (32 * s2 + 8 * g))
                                    : u32x4{0u, 0u, 0u, 0u};
        }
    };

    // chunk 0 into the first buffer while each wave reads its 16 heads' queries into the
    // B operands (channels 32 st + 8 g .. of head j) from the second, which chunk 1
    // overwrites only after the barrier that every wave reaches after these reads
    if (nch > 0) issue(0);
    u32x4 qv[NQ];
    {
        const uint8_t* qh = Q + (16 * hs + j) * gd::kQStride + 16 * g;
#pragma unroll
        for (int st = 0; st < NQ; ++st) qv[st] = *reinterpret_cast<const u32x4*>(qh + 64 * st);
    }
    f32x4 o[2][4];                                         // head tile t, value channels 64 w + 16 mt ..
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) o[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float M[2] = {kNegInf, kNegInf};                       // running maxima of head j of each tile (base 2)
    float sloc = 0.0f;                                     // the lane's sum over its QK rows (head tile hs)
    float* Ph = P + (16 * hs + j) * gd2::kPStride;
    for (int c = 0; c < nch; ++c) {
        zm_c = zm_n;
        if constexpr (kRope) {
            rope_c[0] = rope_n[0];
            rope_c[1] = rope_n[1];
        }
        uint8_t* Vb = V + (c & 1) * gd2::kBuf;
        wait_vmcnt<0>();                                   // chunk c landed
        if (__builtin_amdgcn_ballot_w64(zm_c != 0u)) {
            for (int i = 0; i < C / 8; ++i)
                if ((zm_c >> i) & 1u) *reinterpret_cast<u32x4*>(Vb + VS * (w + 8 * i) + 16 * lane) = u32x4{0u, 0u, 0u, 0u};
        }
        __syncthreads();                                   // its rows; every wave is done with chunk c - 1
        if (c + 1 < nch) issue(c + 1);                     // into chunk c - 1's buffer

        // ---- QK: the wave's row tile of the chunk for its 16 heads
        const int base = C * chunk_of(c);
        const int nc = (n - base < C) ? n - base : C;
        const bool live = 16 * wq < nc;
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        if (live) {
            const uint8_t* krow = Vb + (16 * wq + j) * VS;
#pragma unroll
            for (int st = 0; st < NMAIN; ++st)
                acc = mfma_bf16(*reinterpret_cast<const u32x4*>(krow + 2 * (32 * st + 8 * g)), qv[st], acc);
            if constexpr (kRope) {
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) acc = mfma_bf16(rope_c[s2], qv[NMAIN + s2], acc);
            }
        }
        float z[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * wq + 4 * g + r;
            z[r] = (live && ridx[base + row] >= 0) ? acc[r] * zscale : kNegInf;
        }

        // ---- the chunk's maximum per head across the head tile's four waves, then P
        float mloc = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 16, 64));
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
        if (g == 0) red[16 * w + j] = mloc;
        lds_barrier();
        // both head tiles' new maxima (every wave accumulates both in PV); what has been
        // accumulated is rescaled to them (nothing yet while a maximum is -inf)
        float alpha[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            float Mn = M[t];
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) Mn = fmaxf(Mn, red[16 * (4 * t + ww) + j]);
            alpha[t] = (Mn == kNegInf) ? 1.0f : __builtin_amdgcn_exp2f(M[t] - Mn);
            M[t] = Mn;
        }
        const float Mh = hs ? M[1] : M[0];
        f32x4 pv4;
        float s4 = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pv4[r] = (z[r] == kNegInf) ? 0.0f : __builtin_amdgcn_exp2f(z[r] - Mh);
            s4 += pv4[r];
        }
        *reinterpret_cast<f32x4*>(Ph + 16 * wq + 4 * g) = pv4;
        sloc = sloc * (hs ? alpha[1] : alpha[0]) + s4;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) o[t][mt][r] *= alpha[t];
        lds_barrier();                                     // the chunk's P

        // ---- PV over the chunk's rows for value channels 64 w .. 64 w + 63 of both head tiles
        // (each V^T operand read once for the pair's 32 heads)
#pragma unroll
        for (int st = 0; st < C / 32; ++st) {
            if (32 * st >= nc) break;
            u32x4 pa[2], pb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float* pr = P + (16 * t + j) * gd2::kPStride + 32 * st + 8 * g;
                const f32x4 p0 = *reinterpret_cast<const f32x4*>(pr), p1 = *reinterpret_cast<const f32x4*>(pr + 4);
                const float p[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
                split_bf16x8(p, pa[t], pb[t]);
            }
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int c0 = 64 * w + 16 * mt;
                const uint8_t* vp = Vb + (32 * st + 8 * g + (j >> 2)) * VS + 2 * (c0 + 4 * (j & 3));
                const u32x2 r0 = ds_tr16(vp), r1 = ds_tr16(vp + 4 * VS);
                const u32x4 av = u32x4{r0.x, r0.y, r1.x, r1.y};
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    o[t][mt] = mfma_bf16(av, pa[t], o[t][mt]);
                    o[t][mt] = mfma_bf16(av, pb[t], o[t][mt]);
                }
            }
        }
    }

    // ---- the split's partials: the wave's value channels of both head tiles
    sloc += __shfl_xor(sloc, 16, 64);
    sloc += __shfl_xor(sloc, 32, 64);
    if (g == 0) red[128 + 16 * w + j] = sloc;
    lds_barrier();
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        float l = red[128 + 16 * (4 * t) + j];
#pragma unroll
        for (int ww = 1; ww < 4; ++ww) l += red[128 + 16 * (4 * t + ww) + j];
        const int head = 32 * hp + 16 * t + j;
        const int64_t prow = ((int64_t)b * S + split) * a.H + head;
        const float f = (l > 0.0f) ? __builtin_amdgcn_rcpf(l) : 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            *reinterpret_cast<float4*>(o_part + prow * kDv + 64 * w + 16 * mt + 4 * g) =
                make_float4(o[t][mt][0] * f, o[t][mt][1] * f, o[t][mt][2] * f, o[t][mt][3] * f);
        if (w == 0 && g == 0)
            lse_part[prow] = (l > 0.0f) ? (M[t] + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : -__builtin_inff();
    }
}

template <int DQK>
__global__ __launch_bounds__(512) void k_decode_pair(DecodeArgs a, int S_main, int S_win, int rps, int rps_win,
                                                     int pairs, int n_items, float* o_part, float* lse_part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int L = blockIdx.x;
    const int per = gridDim.x >> 3;
    const int item = (L & 7) * per + (L >> 3);
    if (item >= n_items) return;
    const int S = S_main + S_win;
    const int hp = item % pairs;
    const int rest = item / pairs;
    const int split = rest % S;
    const int b = rest / S;
    if (split < S_main) {
        const int64_t first = (int64_t)split * rps;
        const int n = (int)((a.k - first < rps) ? a.k - first : rps);
        decode_split_pair<DQK>(a, smem, b, split, S, hp, false, first, n, o_part, lse_part);
    } else {
        const int64_t first = (int64_t)(split - S_main) * rps_win;
        const int wl = (int)clamp_visible(a.win_len[b], a.W);
        int n = (int)(wl - first);
        n = n < 0 ? 0 : (n > rps_win ? rps_win : n);
        decode_split_pair<DQK>(a, smem, b, split, S, hp, true, first, n, o_part, lse_part);
    }
}

template <int SRC_MAIN, int DQK>
__global__ __launch_bounds__(512) void k_decode_g(DecodeArgs a, int S_main, int S_win, int rps, int rps_win,
                                                  int groups, int n_items, float* o_part, float* lse_part) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int L = blockIdx.x;
    const int per = gridDim.x >> 3;
    const int item = (L & 7) * per + (L >> 3);
    if (item >= n_items) return;
    const int S = S_main + S_win;
    const int hg = item % groups;
    const int rest = item / groups;
    const int split = rest % S;
    const int b = rest / S;
    constexpr int RM = SRC_MAIN == SRC_E4M3 ? 256 : 128;
    if (split < S_main) {
        const int64_t first = (int64_t)split * rps;
        const int n = (int)((a.k - first < rps) ? a.k - first : rps);
        decode_split_g<SRC_MAIN, DQK, RM>(a, smem, b, split, S, hg, false, first, n, rps, o_part, lse_part);
    } else {
        const int64_t first = (int64_t)(split - S_main) * rps_win;
        const int wl = (int)clamp_visible(a.win_len[b], a.W);
        int n = (int)(wl - first);
        n = n < 0 ? 0 : (n > rps_win ? rps_win : n);
        if constexpr (DQK == 512) {
            if (a.win8) {                                  // MXFP8 entries, widened as they are staged
                decode_split_g<SRC_MX8, DQK, 128>(a, smem, b, split, S, hg, true, first, n, rps_win, o_part,
                                                  lse_part);
                return;
            }
        }
        decode_split_g<SRC_BF16, DQK, 128>(a, smem, b, split, S, hg, true, first, n, rps_win, o_part, lse_part);
    }
}

// Combine the splits of one (b, h) by their logsumexp; thread t owns channels 4t .. 4t+3.
// Up to NF splits (4, 8, 12 or kMergeFast: the launcher's fewest that cover S), every
// load (logsumexps and partials) is issued at once, from clamped in-bounds
// addresses, so the block pays one memory round trip.
// With attention sinks the head's sink logit joins the normaliser (no value
// vector): out scales by exp(lse_U - lse) and lse = logaddexp(lse_U, sink).
// The output's RoPE inverse on thread t's four channels 4t .. 4t + 3 (the
// trailing r channels: halves x1, x2 of r / 2 each, pair i = (x1[i], x2[i])
// becomes (x1 cos + x2 sin, x2 cos - x1 sin)); the partner channel sits r / 8
// lanes away in the same wave (r <= 256 keeps the trailing channels in the
// last wave of the 128 threads). Every lane of the wave takes part in the shuffle.
__device__ __forceinline__ float4 unrotate4(float4 v, int t, int r, const float* cs) {
    const int c0 = 4 * t, base = kDv - r, half = r / 2;
    const bool in = r > 0 && c0 >= base;
    const bool first = c0 < base + half;
    const int lane = t & 63, dl = half / 4;
    const int src = in ? (first ? lane + dl : lane - dl) : lane;
    float4 p;
    p.x = __shfl(v.x, src, 64);
    p.y = __shfl(v.y, src, 64);
    p.z = __shfl(v.z, src, 64);
    p.w = __shfl(v.w, src, 64);
    if (!in) return v;
    const int i0 = (c0 - base) % half;                    // pair of the first channel
    float c[4], s[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        c[e] = cs[2 * (i0 + e)];
        s[e] = cs[2 * (i0 + e) + 1];
    }
    if (first)
        return make_float4(v.x * c[0] + p.x * s[0], v.y * c[1] + p.y * s[1], v.z * c[2] + p.z * s[2],
                           v.w * c[3] + p.w * s[3]);
    return make_float4(v.x * c[0] - p.x * s[0], v.y * c[1] - p.y * s[1], v.z * c[2] - p.z * s[2],
                       v.w * c[3] - p.w * s[3]);
}

__device__ __forceinline__ void merge_finish(float m, float tot, float4 acc, const float* sinks, int h, float4* o,
                                            float* lse_out, int t, int r, const float* cs) {
    if (sinks) {
        const float sk = sinks[h];
        if (sk > -__builtin_inff()) {
            const float M = fmaxf(m, sk), f = __expf(m - M);
            tot = tot * f + __expf(sk - M);
            acc = make_float4(acc.x * f, acc.y * f, acc.z * f, acc.w * f);
            m = M;
        }
    }
    const float inv = 1.0f / tot;
    float4 v = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (r > 0) v = unrotate4(v, t, r, cs);
    *o = v;
    if (t == 0) *lse_out = m + __logf(tot);
}

template <int NF>
__global__ __launch_bounds__(kMergeThreads) void k_merge(int S, int H, const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part, float* __restrict__ out,
                                                         float* __restrict__ lse, const float* __restrict__ sinks,
                                                         int rope_dim, const float* __restrict__ rope_cs) {
    static_assert(NF >= 1 && NF <= kMergeFast, "splits loaded in one round");
    const int h = blockIdx.x, b = blockIdx.y;
    const int t = threadIdx.x;
    const float* lp = lse_part + (int64_t)b * S * H + h;
    // an empty set: all mass on the sink (lse = the sink's logit, -inf without one)
    const float empty_lse = sinks ? sinks[h] : -__builtin_inff();
    const float* cs = rope_dim > 0 ? rope_cs + (int64_t)b * rope_dim : nullptr;   // [r / 2][2] of sequence b
    if (S <= NF) {
        const float4* op = reinterpret_cast<const float4*>(o_part + ((int64_t)b * S * H + h) * kDv) + t;
        const int64_t step = (int64_t)H * (kDv / 4);
        float lv[NF];
        float4 pv[NF];
#pragma unroll
        for (int s = 0; s < NF; ++s) {
            const int sc = (s < S) ? s : 0;
            lv[s] = lp[(int64_t)sc * H];
            pv[s] = op[sc * step];
        }
        float m = -__builtin_inff();
#pragma unroll
        for (int s = 0; s < NF; ++s)
            if (s < S) m = fmaxf(m, lv[s]);
        float4* o = reinterpret_cast<float4*>(out + ((int64_t)b * H + h) * kDv) + t;
        if (m == -__builtin_inff()) {
            *o = make_float4(0.f, 0.f, 0.f, 0.f);
            if (t == 0) lse[(int64_t)b * H + h] = empty_lse;
            return;
        }
        float tot = 0.0f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int s = 0; s < NF; ++s) {
            const float wv = (s < S) ? __expf(lv[s] - m) : 0.0f;
            tot += wv;
            acc.x += wv * pv[s].x;
            acc.y += wv * pv[s].y;
            acc.z += wv * pv[s].z;
            acc.w += wv * pv[s].w;
        }
        merge_finish(m, tot, acc, sinks, h, o, &lse[(int64_t)b * H + h], t, rope_dim, cs);
        return;
    }
    float m = -__builtin_inff();
    for (int s = 0; s < S; ++s) m = fmaxf(m, lp[(int64_t)s * H]);
    float4* o = reinterpret_cast<float4*>(out + ((int64_t)b * H + h) * kDv) + t;
    if (m == -__builtin_inff()) {
        *o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t == 0) lse[(int64_t)b * H + h] = empty_lse;
        return;
    }
    const float4* op = reinterpret_cast<const float4*>(o_part + ((int64_t)b * S * H + h) * kDv) + t;
    const int64_t step = (int64_t)H * (kDv / 4);
    float tot = 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
        const float wv = __expf(lp[(int64_t)s * H] - m);
        const float4 v = op[s * step];
        tot += wv;
        acc.x += wv * v.x;
        acc.y += wv * v.y;
        acc.z += wv * v.z;
        acc.w += wv * v.w;
    }
    merge_finish(m, tot, acc, sinks, h, o, &lse[(int64_t)b * H + h], t, rope_dim, cs);
}

// ------------------------------------------------------------------------
// Generic path.
__device__ __forceinline__ float e2m1_val(uint32_t n) {
    const uint32_t e = (n >> 1) & 3u, m = n & 1u;
    const float mag = e ? __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)e - 1) : 0.5f * (float)m;
    return (n & 8u) ? -mag : mag;
}

__device__ __forceinline__ float row_elem(int fmt, int dim, const uint8_t* row, int c) {
    switch (fmt) {
    case MLA_FMT_F32: return reinterpret_cast<const float*>(row)[c];
    case MLA_FMT_BF16: return u2f((uint32_t)reinterpret_cast<const uint16_t*>(row)[c] << 16);
    case MLA_FMT_E4M3_S128:
        if (c < dim) return e4m3_to_f32(row[c]) * reinterpret_cast<const float*>(row + dim)[c / 128];
        return u2f((uint32_t)reinterpret_cast<const uint16_t*>(row + dim + 4 * (dim / 128))[c - dim] << 16);
    case MLA_FMT_MXFP4: {
        const uint32_t byte = row[c / 2];
        return e2m1_val((c & 1) ? (byte >> 4) : (byte & 15u)) * e8m0_to_f32(row[dim / 2 + c / 32]);
    }
    default: {
        const uint32_t byte = row[c / 2];
        return e2m1_val((c & 1) ? (byte >> 4) : (byte & 15u)) * e4m3_to_f32(row[dim / 2 + c / 16]);
    }
    }
}

__global__ __launch_bounds__(kGenericThreads) void k_decode_generic(DecodeArgs a) {
    __shared__ float zs[kGenericMaxRows];
    __shared__ float qs[1024];
    __shared__ float os[1024];
    __shared__ float red[kGenericThreads / 64];
    const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int D = a.dim + a.rope;
    const int n = a.k + (a.win ? a.W : 0);
    for (int c = t; c < D; c += kGenericThreads)
        qs[c] = (a.fmt == MLA_FMT_F32)
                    ? reinterpret_cast<const float*>(a.q)[((int64_t)b * a.H + h) * D + c]
                    : u2f((uint32_t)reinterpret_cast<const uint16_t*>(a.q)[((int64_t)b * a.H + h) * D + c] << 16);
    __syncthreads();
    auto src = [&](int u, bool* win) -> const uint8_t* {
        *win = u >= a.k;
        if (!*win) {
            const int32_t s = a.idx[(int64_t)b * a.k + u];
            if (s < 0 || s >= a.capacity) return nullptr;
            return a.cache + b * a.stride + (int64_t)s * a.row_bytes;
        }
        const int slot = u - a.k;
        if (slot >= clamp_visible(a.win_len[b], a.W)) return nullptr;
        return reinterpret_cast<const uint8_t*>(a.win + ((int64_t)b * a.W + slot) * D);
    };
    float mx = -__builtin_inff();
    for (int u = t; u < n; u += kGenericThreads) {
        bool win;
        const uint8_t* r = src(u, &win);
        float z = -__builtin_inff();
        if (r) {
            float d = 0.0f;
            for (int c = 0; c < D; ++c)
                d += qs[c] * (win ? u2f((uint32_t)reinterpret_cast<const uint16_t*>(r)[c] << 16)
                                  : row_elem(a.fmt, a.dim, r, c));
            z = d * a.scale;
        }
        zs[u] = z;
        mx = fmaxf(mx, z);
    }
    mx = wave_max(mx);
    if ((t & 63) == 0) red[t >> 6] = mx;
    __syncthreads();
    mx = red[0];
    for (int i = 1; i < kGenericThreads / 64; ++i) mx = fmaxf(mx, red[i]);
    const float sink = a.sinks ? a.sinks[h] : -__builtin_inff();   // the sink column's logit
    mx = fmaxf(mx, sink);
    __syncthreads();
    float* o = a.out + ((int64_t)b * a.H + h) * a.d_v;
    if (mx == -__builtin_inff()) {
        for (int c = t; c < a.d_v; c += kGenericThreads) o[c] = 0.0f;
        if (t == 0) a.lse[(int64_t)b * a.H + h] = -__builtin_inff();
        return;
    }
    float sum = 0.0f;
    for (int u = t; u < n; u += kGenericThreads) {
        const float p = __expf(zs[u] - mx);
        zs[u] = p;
        sum += p;
    }
    sum = wave_sum(sum);
    if ((t & 63) == 0) red[t >> 6] = sum;
    __syncthreads();
    sum = 0.0f;
    for (int i = 0; i < kGenericThreads / 64; ++i) sum += red[i];
    if (sink > -__builtin_inff()) sum += __expf(sink - mx);
    for (int c = t; c < a.d_v; c += kGenericThreads) {
        float acc = 0.0f;
        for (int u = 0; u < n; ++u) {
            const float p = zs[u];
            if (p == 0.0f) continue;
            bool win;
            const uint8_t* r = src(u, &win);
            acc += p * (win ? u2f((uint32_t)reinterpret_cast<const uint16_t*>(r)[c] << 16)
                            : row_elem(a.fmt, a.dim, r, c));
        }
        os[c] = acc / sum;
    }
    __syncthreads();
    // the output's RoPE inverse on the trailing rope_dim channels (pair i: x1 = os[base + i],
    // x2 = os[base + r/2 + i] -> x1 cos + x2 sin, x2 cos - x1 sin)
    const int r = a.rope_dim, base = a.d_v - r, half = r / 2;
    const float* cs = r > 0 ? a.rope_cs + (int64_t)b * r : nullptr;
    for (int c = t; c < a.d_v; c += kGenericThreads) {
        float v = os[c];
        if (r > 0 && c >= base) {
            const int i = (c - base) % half;
            const float cv = cs[2 * i], sv = cs[2 * i + 1];
            v = (c < base + half) ? os[c] * cv + os[c + half] * sv : os[c] * cv - os[c - half] * sv;
        }
        o[c] = v;
    }
    if (t == 0) a.lse[(int64_t)b * a.H + h] = mx + __logf(sum);
}

bool mfma_shape(int fmt, int dim, int rope, int d_v, int H) {
    if (d_v != kDv || (H != 16 && H != 32 && H != 64 && H != 128)) return false;
    if (fmt == MLA_FMT_E4M3_S128) return dim == 512 && rope == 64;
    if (fmt == MLA_FMT_E2M1_S16) return dim == 512 && rope == 0;
    if (fmt == MLA_FMT_BF16) return dim == 512 && (rope == 64 || rope == 0);
    return false;
}

}  // namespace

bool decode_supported(int fmt, int dim, int rope, int d_v, int H) {
    if (mfma_shape(fmt, dim, rope, d_v, H)) return true;
    return dim + rope <= 1024 && d_v <= dim + rope && d_v > 0;
}

struct Geometry {
    int groups, rps, rps_win, S_main, S_win;
};

// Splits of the gather-all decode: R = 256 rows for E4M3 rows, 128 otherwise (and for
// the window), halved (down to 32) while the chip is short of a workgroup per CU, the
// halved splits still fit one round of workgroups (one per CU: the LDS holds one) and
// the merge still takes every split's partial in one round of loads (kMergeFast);
// the option decode_rows_per_split (32 .. R, a multiple of 32) overrides the main rows' R.
Geometry gather_geometry(int fmt, int B, int H, int k, int W) {
    Geometry g{};
    g.groups = H / 16;
    const int R = fmt == MLA_FMT_E4M3_S128 ? 256 : 128;
    int rps = R, rpw = 128;
    const int v = (int)option(OPT_DECODE_RPS);
    if (v >= 32 && v <= R && v % 32 == 0) {
        rps = v;
    } else {
        auto blocks = [&](int r, int rw) {
            return (int64_t)B * g.groups * ((k + r - 1) / r + (W + rw - 1) / rw);
        };
        auto splits = [&](int r, int rw) { return (k + r - 1) / r + (W + rw - 1) / rw; };
        while (rps > 32 && blocks(rps, rpw) < 256 && blocks(rps / 2, rpw > 32 ? rpw / 2 : rpw) <= 256 &&
               splits(rps / 2, rpw > 32 ? rpw / 2 : rpw) <= kMergeFast) {
            rps /= 2;
            if (rpw > 32) rpw /= 2;
        }
    }
    g.rps = rps;
    g.rps_win = rpw;
    g.S_main = (k + rps - 1) / rps;
    g.S_win = (W + rpw - 1) / rpw;
    return g;
}

// Two head tiles per workgroup for bf16 rows when one head tile per workgroup would
// take more than one round of the CUs: each row is then staged once per 32 heads.
static bool use_pairs(int fmt, int B, int H, const Geometry& g) {
    return fmt == MLA_FMT_BF16 && H % 32 == 0 && (int64_t)B * (g.S_main + g.S_win) * g.groups > 256;
}

// Splits of the paired decode, which streams its rows in chunks of 64: the fewest
// rows per split (64 .. 512, doubling) that keep the grid within one round of
// workgroups (one per CU), else 512; 128 window slots per split. The option
// decode_rows_per_split, when a multiple of 64, overrides the main rows per split.
static Geometry pair_geometry(int B, int H, int k, int W) {
    Geometry g{};
    g.groups = H / 32;
    int rps = 64;
    const int rpw = 128;
    const int v = (int)option(OPT_DECODE_RPS);
    const int64_t S_win = (W + rpw - 1) / rpw;
    if (v >= 64 && v <= 512 && v % 64 == 0) {
        rps = v;
    } else {
        while (rps < 512 && (int64_t)B * g.groups * ((k + rps - 1) / rps + S_win) > 256) rps *= 2;
    }
    g.rps = rps;
    g.rps_win = rpw;
    g.S_main = (k + rps - 1) / rps;
    g.S_win = (int)S_win;
    return g;
}

// The splits the MFMA decode runs with (pairs: whether it pairs head tiles).
static Geometry decode_geometry(int fmt, int B, int H, int k, int W, bool* pairs) {
    const Geometry g = gather_geometry(fmt, B, H, k, W);
    *pairs = use_pairs(fmt, B, H, g);
    return *pairs ? pair_geometry(B, H, k, W) : g;
}

size_t decode_workspace_bytes(int fmt, int dim, int rope, int d_v, int B, int H, int k, int W) {
    if (!mfma_shape(fmt, dim, rope, d_v, H)) return 0;
    bool pairs = false;
    const Geometry g = decode_geometry(fmt, B, H, k, W, &pairs);
    const size_t S = (size_t)(g.S_main + g.S_win);
    const size_t o = (size_t)B * S * H * kDv * sizeof(float);
    const size_t l = (size_t)B * S * H * sizeof(float);
    return ((o + 255) & ~(size_t)255) + ((l + 255) & ~(size_t)255);
}

template <int SRC_MAIN, int DQK>
static hipError_t launch_gather(const DecodeArgs& a, const Geometry& g, float* o_part, float* lse_part,
                                hipStream_t stream) {
    const int S = g.S_main + g.S_win;
    const int n_items = a.B * S * g.groups;
    const int grid = (n_items + 7) / 8 * 8;
    constexpr int lds = gd::lds_bytes<SRC_MAIN, DQK>();
    auto kern = k_decode_g<SRC_MAIN, DQK>;
    static bool attr_set = false;                          // dynamic LDS above 64 KiB, once per kernel
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const ProfSlot p = prof_slot(PROF_DECODE);
    return launch_kernel(kern, dim3(grid), dim3(512), lds, stream, p.start, p.stop, a, g.S_main, g.S_win, g.rps,
                         g.rps_win, g.groups, n_items, o_part, lse_part);
}

template <int DQK>
static hipError_t launch_pair(const DecodeArgs& a, const Geometry& g, float* o_part, float* lse_part,
                              hipStream_t stream) {
    const int S = g.S_main + g.S_win;
    const int pairs = a.H / 32;
    const int n_items = a.B * S * pairs;
    const int grid = (n_items + 7) / 8 * 8;
    auto kern = k_decode_pair<DQK>;
    static bool attr_set = false;                          // dynamic LDS above 64 KiB, once per kernel
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, gd2::kBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const ProfSlot p = prof_slot(PROF_DECODE);
    return launch_kernel(kern, dim3(grid), dim3(512), gd2::kBytes, stream, p.start, p.stop, a, g.S_main, g.S_win,
                         g.rps, g.rps_win, pairs, n_items, o_part, lse_part);
}

// An MXFP8 window ring [B, W, D + D/32 bytes] widened to bf16 rows [B, W, D]:
// the E4M3 value times its block's power of two, formed in fp32 (exact) and
// rounded to bf16, exact unless the product lies below bf16's smallest
// subnormal (blocks with a scale code below 3). One workgroup per ring slot.
__global__ __launch_bounds__(256) void k_widen_window(const uint8_t* __restrict__ ring, int D,
                                                      uint16_t* __restrict__ out) {
    const int64_t row = blockIdx.x;
    const uint8_t* src = ring + row * (D + D / 32);
    for (int c = threadIdx.x; c < D; c += 256)
        out[row * D + c] = (uint16_t)bf16_rne(e4m3_to_f32(src[c]) * e8m0_to_f32(src[D + c / 32]));
}

bool decode_takes_select_lists(int fmt, int dim, int rope, int d_v, int B, int H, int k, int W) {
    (void)B;
    (void)W;
    return mfma_shape(fmt, dim, rope, d_v, H) && k > 0;
}

bool decode_fuses_window_append(const DecodeArgs& a) {
    if (!a.new_win || !a.win_pos || a.W <= 0 || (!a.win && !a.win8) || a.B <= 0) return false;
    if (!mfma_shape(a.fmt, a.dim, a.rope, a.d_v, a.H) || a.dim + a.rope != 512) return false;
    if (reinterpret_cast<uintptr_t>(a.new_win) % 16 != 0) return false;
    if (use_pairs(a.fmt, a.B, a.H, gather_geometry(a.fmt, a.B, a.H, a.k, a.W))) return false;
    return reinterpret_cast<uintptr_t>(a.win8 ? static_cast<const void*>(a.win8) : a.win) % 16 == 0;
}

hipError_t launch_decode(const DecodeArgs& a_in, hipStream_t stream) {
    if (a_in.B == 0) return hipSuccess;
    DecodeArgs a = a_in;
    // MXFP8 window entries of 512 channels (16-byte aligned) are widened inside the gather
    // decode's staging; others are first widened to a bf16 copy after the decode's own workspace
    const bool mfma = mfma_shape(a.fmt, a.dim, a.rope, a.d_v, a.H);
    bool pairs = false;
    const Geometry g = decode_geometry(a.fmt, a.B, a.H, a.k, (a.win || a.win8) ? a.W : 0, &pairs);
    pairs = pairs && mfma;
    const bool win8_inline = a.win8 && mfma && !pairs && a.dim + a.rope == 512 &&
                             reinterpret_cast<uintptr_t>(a.win8) % 16 == 0;
    if (a.win8 && a.W > 0 && !win8_inline) {
        const size_t base = decode_workspace_bytes(a.fmt, a.dim, a.rope, a.d_v, a.B, a.H, a.k, a.W);
        uint16_t* wide = reinterpret_cast<uint16_t*>(static_cast<char*>(a.workspace) + base);
        const hipError_t e = launch_kernel(k_widen_window, dim3((unsigned)(a.B * a.W)), dim3(256), 0, stream,
                                           nullptr, nullptr, a.win8, a.dim + a.rope, wide);
        if (e != hipSuccess) return e;
        a.win = wide;
        a.win8 = nullptr;
    }
    if (!mfma) {
        const ProfSlot p = prof_slot(PROF_DECODE);
        return launch_kernel(k_decode_generic, dim3(a.H, a.B), dim3(kGenericThreads), 0, stream, p.start, p.stop, a);
    }
    const int S = g.S_main + g.S_win;
    const size_t o_bytes = (((size_t)a.B * S * a.H * kDv * sizeof(float)) + 255) & ~(size_t)255;
    float* o_part = reinterpret_cast<float*>(a.workspace);
    float* lse_part = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + o_bytes);
    if (S > 0) {
        hipError_t e = hipSuccess;
        if (a.fmt == MLA_FMT_E4M3_S128) e = launch_gather<SRC_E4M3, 576>(a, g, o_part, lse_part, stream);
        else if (a.fmt == MLA_FMT_E2M1_S16) e = launch_gather<SRC_FP4, 512>(a, g, o_part, lse_part, stream);
        else if (pairs) e = a.rope == 64 ? launch_pair<576>(a, g, o_part, lse_part, stream)
                                         : launch_pair<512>(a, g, o_part, lse_part, stream);
        else if (a.rope == 64) e = launch_gather<SRC_BF16, 576>(a, g, o_part, lse_part, stream);
        else e = launch_gather<SRC_BF16, 512>(a, g, o_part, lse_part, stream);
        if (e != hipSuccess) return e;
    }
    // the merge's one-round path loads the fewest splits (4, 8, 12 or 16) that cover S
    const ProfSlot p = prof_slot(PROF_MERGE);
    auto merge = S <= 4 ? k_merge<4> : S <= 8 ? k_merge<8> : S <= 12 ? k_merge<12> : k_merge<kMergeFast>;
    return launch_kernel(merge, dim3(a.H, a.B), dim3(kMergeThreads), 0, stream, p.start, p.stop, S, a.H, o_part,
                         lse_part, a.out, a.lse, a.sinks, a.rope_dim, a.rope_cs);
}

}  // namespace mla
