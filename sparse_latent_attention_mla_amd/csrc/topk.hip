// topk.hip -- exact top-k over the indexer scores.
//
// Selection ([P1] "DeepSeek's Attention and KV Cache - From MLA to CSA2",
// "DeepSeek-V3.2", eq. 2; [P2] "From MLA to DSA to HCA/CSA", Part 1): the k
// visible rows of largest score, ties at the k-th score going to the smaller
// position; slots past min(k, n_visible) hold -1 ([P2] "CSA: two changes to
// HCA").  Radix selection on order-preserving score keys:
//   1. the scan kernel has built a histogram of the top kHistBits key bits;
//   2. k_select (many workgroups per sequence) finds the bin T holding the
//      k-th largest key, and each workgroup compacts, in LDS, the rows of its
//      slice that lie above T (selected) and in T (candidates, as 64-bit
//      key << 32 | ~position) and writes both lists and their counts to its
//      own slots (no global atomics: across XCDs they serialise);
//   3. k_select_final (one workgroup per sequence) prefix-sums the counts,
//      gathers the selected positions into the output and the candidates
//      into one list, then radix-selects the missing
//      count among the candidates, most significant digit first: two 10-bit
//      digits fix the exact threshold score (the bin fixed the top 12 of its 32
//      bits); only when more rows share that score than are still needed do
//      four 8-bit digits of the inverted position follow, so the smaller
//      position wins a tie. It then pads with -1. (A separate launch: handing
//      the lists over inside one kernel needs a device-scope fence in every
//      workgroup, which costs more than the launch.)
// Sequences of up to kRowPathMax rows take a shorter path: one workgroup per
// sequence reads every score, finds T, appends every row of bin T or above to
// one LDS list (one compare and one ballot per score) and radix-selects in it,
// the rows above T first, with no hand-over between workgroups. (Longer
// sequences outgrow one CU's vector throughput: 64K scores already take it
// longer than the two-kernel path.) The final kernel for more than 64 select
// workgroups, or for selections of blocks, gathers the lists flat
// (k_select_final2_flat).
// Output positions form an unordered set.
// The same kernels select over a candidate pool (the entries of a Reindex
// layer's pool: each selected entry is reported as its position, entries that
// name no visible position as -1, ties going to the smaller position) and over
// block scores (the pool of the hierarchical indexer: each selected block is
// written as its positions); see SelectMap.
#include <cstdlib>

#include "common.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace mla {

namespace {

constexpr int kSelThreads = 256;          // multi-workgroup path
constexpr int kSelRows = kSelRowsHost;    // rows per k_select workgroup
constexpr int kRowThreads = 1024;         // one workgroup per sequence
constexpr int64_t kRowPathMax = 16384;    // longest sequence on the one-workgroup path
constexpr int kFinalLds = 6144;           // candidates kept in LDS (48 KB)

// One sequence's output row: reported value v goes to slot o as v itself, or,
// expanding blocks of `expand` positions, as v * expand + j in slots
// o * expand + j (-1 as -1s).
// (EXPAND false: expand is 1, and the kernels compile to plain stores.)
template <bool EXPAND>
struct OutRow {
    int32_t* out;
    int expand;
    __device__ __forceinline__ void put(uint32_t o, int32_t v) const {
        if constexpr (!EXPAND) {
            out[o] = v;
        } else {
            for (int j = 0; j < expand; ++j) out[(int64_t)o * expand + j] = v < 0 ? -1 : v * expand + j;
        }
    }
};
template <bool EXPAND>
__device__ __forceinline__ OutRow<EXPAND> out_row(int32_t* out_idx, int b, int k, const SelectMap& m) {
    return OutRow<EXPAND>{out_idx + (int64_t)b * k * (EXPAND ? m.expand : 1), EXPAND ? m.expand : 1};
}

// Sequence b's view of a SelectMap: the position entry s reports, given the
// pool entry cv = cand[b, s] (loaded with the score; unused without a pool).
template <bool POOL>
struct PosMap {
    int64_t lim;
    __device__ __forceinline__ int32_t operator()(int64_t s, int32_t cv) const {
        if constexpr (!POOL) return (int32_t)s;
        else return (cv >= 0 && cv < lim) ? cv : -1;
    }
};
template <bool POOL>
__device__ __forceinline__ PosMap<POOL> pos_map(const SelectMap& m, int b) {
    return PosMap<POOL>{POOL ? clamp_visible(m.n_visible[b], m.limit) : 0};
}
__device__ __forceinline__ int64_t visible_of(const int32_t* n_visible, int b, int64_t capacity) {
    return n_visible ? clamp_visible(n_visible[b], capacity) : capacity;
}

// The list c[0 .. ncand) (64-bit key << 32 | ~position) holds entries whose
// top-12-bit bin is T (nT of them) or, when `above` is set, above T. Append to
// out from the LDS cursor on every entry above bin T and the positions of the
// `need` largest of bin T (entries at or past `want` are not written). Two
// 10-bit digits fix the exact threshold score; only when more entries share it
// than are still needed do four 8-bit digits of the inverted position follow.
// h: two LDS histograms of kMaxDigitBins, the first zero on entry; res: 4 LDS words.
template <int NT, typename P, typename OUT>
__device__ void radix_take_bins(P c, uint32_t ncand, int T, uint32_t nT, bool above, uint32_t need, uint32_t want,
                                OUT out, uint32_t* cursor, uint32_t (*h)[kMaxDigitBins], uint32_t* res) {
    const int t = threadIdx.x, lane = t & 63;
    const bool radix = need > 0 && need < nT;
    uint64_t prefix = (uint64_t)(uint32_t)T << 52, mask = 0xFFFull << 52;
    uint32_t rem = need;
    int par = 0;
    auto pass = [&](int shift, int bits) {
        const int nb = 1 << bits;
        uint32_t* hc = h[par];
        for (uint32_t i = t; i < ncand; i += NT) {
            const uint64_t v = c[i];
            if ((v & mask) == prefix) atomicAdd(&hc[(v >> shift) & (uint64_t)(nb - 1)], 1u);
        }
        lds_barrier();
        if (t < 64) {                                    // one wave finds the digit
            const DigitResult r = wave_find_digit(hc, nb, rem);
            if (lane == 0) {
                res[0] = (uint32_t)r.digit;
                res[1] = r.above;
                res[2] = r.count;
            }
        } else {                                         // the others clear the next histogram
            for (int i = t - 64; i < kMaxDigitBins; i += NT - 64) h[par ^ 1][i] = 0u;
        }
        lds_barrier();
        const int d = (int)res[0];
        prefix |= (uint64_t)d << shift;
        mask |= (uint64_t)(nb - 1) << shift;
        rem -= res[1];
        par ^= 1;
        return res[2];                                   // entries sharing the prefix so far
    };
    if (radix) {
        pass(42, 10);
        const uint32_t eq = pass(32, 10);                // prefix now holds the exact threshold score
        if (rem < eq) {                                  // ties at that score: smaller positions first
            pass(24, 8);
            pass(16, 8);
            pass(8, 8);
            pass(0, 8);
        }
    }
    // the entries above bin T first, then those of bin T at or above the prefix:
    // exactly `need` of them, above the threshold score and at it either all (score
    // resolved, count fits) or those above the exact composite (need == nT: all).
    // (Equal composites, which only entries reported as -1 share, may exceed `need`;
    // the excess lands past `want` and is dropped, after every entry above bin T.)
    const uint64_t binT = (uint64_t)(uint32_t)T;
    const uint32_t n_iter = (ncand + NT - 1) / NT;
    auto take_pass = [&](bool of_t) {
        for (uint32_t it = 0; it < n_iter; ++it) {
            const uint32_t i = it * NT + t;
            bool take = false;
            int32_t pos = 0;
            if (i < ncand) {
                const uint64_t v = c[i];
                take = of_t ? ((v >> 52) == binT && v >= prefix) : (v >> 52) > binT;
                pos = (int32_t)(~(uint32_t)(v & 0xFFFFFFFFull));
            }
            const uint64_t m = __ballot(take);
            uint32_t base = 0;
            if (lane == 0 && m) base = atomicAdd(cursor, (uint32_t)__popcll(m));
            base = __shfl(base, 0, 64);
            if (take) {
                const uint32_t o = base + lanes_below(m);
                if (o < want) out.put(o, pos);
            }
        }
    };
    if (above) {
        take_pass(false);
        lds_barrier();                                   // (the cursor)
    }
    if (need > 0) take_pass(true);
}

// Among the candidates c[0 .. ncand) (all in one top-12-bit bin), append the
// positions of the `need` largest to out from the LDS cursor on: the same radix
// passes over a list that holds bin T only (a separate function: folding it into
// radix_take_bins cost the two-kernel selection 1.5 us per call, measured).
template <int NT, typename P, typename OUT>
__device__ void radix_take(P c, uint32_t ncand, uint32_t need, uint32_t want, OUT out,
                           uint32_t* cursor, uint32_t (*h)[kMaxDigitBins], uint32_t* res) {
    const int t = threadIdx.x, lane = t & 63;
    const bool radix = need > 0 && need < ncand;
    uint64_t prefix = radix ? (c[0] & (0xFFFull << 52)) : 0ull, mask = 0xFFFull << 52;
    uint32_t rem = need;
    int par = 0;
    auto pass = [&](int shift, int bits) {
        const int nb = 1 << bits;
        uint32_t* hc = h[par];
        for (uint32_t i = t; i < ncand; i += NT) {
            const uint64_t v = c[i];
            if ((v & mask) == prefix) atomicAdd(&hc[(v >> shift) & (uint64_t)(nb - 1)], 1u);
        }
        lds_barrier();
        if (t < 64) {                                    // one wave finds the digit
            const DigitResult r = wave_find_digit(hc, nb, rem);
            if (lane == 0) {
                res[0] = (uint32_t)r.digit;
                res[1] = r.above;
                res[2] = r.count;
            }
        } else {                                         // the others clear the next histogram
            for (int i = t - 64; i < kMaxDigitBins; i += NT - 64) h[par ^ 1][i] = 0u;
        }
        lds_barrier();
        const int d = (int)res[0];
        prefix |= (uint64_t)d << shift;
        mask |= (uint64_t)(nb - 1) << shift;
        rem -= res[1];
        par ^= 1;
        return res[2];                                   // candidates sharing the prefix so far
    };
    if (radix) {
        pass(42, 10);
        const uint32_t eq = pass(32, 10);                // prefix now holds the exact threshold score
        if (rem < eq) {                                  // ties at that score: smaller positions first
            pass(24, 8);
            pass(16, 8);
            pass(8, 8);
            pass(0, 8);
        }
    }
    // "v >= prefix" takes exactly `need`: every candidate above the threshold score,
    // and at it either all (score resolved, count fits) or those above the exact composite
    if (need > 0) {
        const uint32_t n_iter = (ncand + NT - 1) / NT;
        for (uint32_t it = 0; it < n_iter; ++it) {
            const uint32_t i = it * NT + t;
            bool take = false;
            int32_t pos = 0;
            if (i < ncand) {
                const uint64_t v = c[i];
                take = !radix || v >= prefix;
                pos = (int32_t)(~(uint32_t)(v & 0xFFFFFFFFull));
            }
            const uint64_t m = __ballot(take);
            uint32_t base = 0;
            if (lane == 0 && m) base = atomicAdd(cursor, (uint32_t)__popcll(m));
            base = __shfl(base, 0, 64);
            if (take) {
                const uint32_t o = base + lanes_below(m);
                if (o < want) out.put(o, pos);
            }
        }
    }
}

struct FinalLds {
    uint64_t lc[kFinalLds];
    uint32_t h[2][kMaxDigitBins];
    uint32_t res[4];
};

// Radix-take over the candidates in LDS (the common case) or in the global list.
template <int NT, typename OUT>
__device__ __forceinline__ void radix_take_any(FinalLds& L, const uint64_t* gc2, uint32_t ncand, uint32_t need,
                                               uint32_t want, OUT out, uint32_t* cursor) {
    if (ncand <= (uint32_t)kFinalLds) radix_take<NT>(L.lc, ncand, need, want, out, cursor, L.h, L.res);
    else radix_take<NT>(gc2, ncand, need, want, out, cursor, L.h, L.res);
}

// Classify one score: above the threshold bin T (take), in it (maybe).
__device__ __forceinline__ void classify(float v, bool in, int T, uint32_t* key, bool* take, bool* maybe) {
    uint32_t kk = 0, bin = 0;
    if (in) {
        kk = score_key(v);
        bin = kk >> (32 - kHistBits);
    }
    *key = kk;
    *take = in && (T < 0 || (int)bin > T);
    *maybe = in && T >= 0 && (int)bin == T;
}

// ---- one workgroup per sequence ------------------------------------------
template <bool POOL, bool EXPAND>
__global__ __launch_bounds__(kRowThreads) void k_topk_row(const float* __restrict__ scores, int64_t capacity,
                                                          const int32_t* __restrict__ n_visible, int k,
                                                          TopkWorkspace ws, int32_t* __restrict__ out_idx,
                                                          SelectMap map) {
    __shared__ FinalLds L;
    __shared__ uint32_t n_hit, cursor, above_s, in_t_s;
    __shared__ int T_s;
    constexpr int kR = 16;                               // scores per thread per round
    constexpr int kRound = kRowThreads * kR;
    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63;
    const int64_t nvis = visible_of(n_visible, b, capacity);
    const uint32_t want = (uint32_t)((nvis < k) ? nvis : k);
    const auto out = out_row<EXPAND>(out_idx, b, k, map);
    const auto pmap = pos_map<POOL>(map, b);
    const int32_t* __restrict__ cb = POOL ? map.cand + b * capacity : nullptr;
    uint64_t* gc2 = ws.cand2 + b * capacity;
    uint32_t* hb = ws.hist + (int64_t)b * kHistWordsHost;
    const float* __restrict__ sc = scores + b * capacity;
    float v[kR];
    int32_t cv[kR];                                      // pool entries (with a pool)
    auto load = [&](int64_t r0) {
#pragma unroll
        for (int u = 0; u < kR; ++u) {
            const int64_t s = r0 + u * kRowThreads + t;
            v[u] = (s < nvis) ? sc[s] : 0.0f;
            if constexpr (POOL) cv[u] = (s < nvis) ? cb[s] : 0;
            else cv[u] = 0;
        }
    };
    load(0);                                             // in flight during the threshold search
    if (t < 64) {
        const DigitResult r = hist_find(hb, (uint32_t)k);
        if (t == 0) {
            T_s = r.found ? r.digit : -1;                // -1: every visible row fits in k
            above_s = r.above;
            in_t_s = r.count;
            n_hit = 0;
            cursor = 0;
        }
    }
    for (int i = t; i < kMaxDigitBins; i += kRowThreads) L.h[0][i] = 0u;
    lds_barrier();
    const int T = T_s;
    if (T < 0) {                                         // every visible entry, in place
        for (int64_t r0 = 0; r0 < nvis; r0 += kRound) {
            if (r0 > 0) load(r0);
#pragma unroll
            for (int u = 0; u < kR; ++u) {
                const int64_t s = r0 + u * kRowThreads + t;
                if (s < nvis) out.put((uint32_t)s, pmap(s, cv[u]));
            }
        }
        zero_hist(hb);
        for (uint32_t i = want + t; i < (uint32_t)k; i += kRowThreads) out.put(i, -1);
        return;
    }
    // the hits: every entry in bin T or above, appended to one list (key << 32 |
    // ~position), one LDS reservation per wave and round
    const uint32_t lo = (uint32_t)T << (32 - kHistBits);
    for (int64_t r0 = 0; r0 < nvis; r0 += kRound) {
        if (r0 > 0) load(r0);
        uint32_t key[kR];
        uint64_t m[kR];
        uint32_t bits = 0, nh = 0;
#pragma unroll
        for (int u = 0; u < kR; ++u) {
            const int64_t s = r0 + u * kRowThreads + t;
            key[u] = score_key(v[u]);
            const bool hit = s < nvis && key[u] >= lo;
            bits |= (uint32_t)hit << u;
            m[u] = __ballot(hit);
            nh += (uint32_t)__popcll(m[u]);
        }
        if (nh) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&n_hit, nh);
            base = __shfl(base, 0, 64);
#pragma unroll
            for (int u = 0; u < kR; ++u) {
                if ((bits >> u) & 1u) {
                    const int64_t s = r0 + u * kRowThreads + t;
                    const uint32_t o = base + lanes_below(m[u]);
                    const uint64_t c = ((uint64_t)key[u] << 32) | (uint64_t)(~(uint32_t)pmap(s, cv[u]));
                    if (o < (uint32_t)kFinalLds) L.lc[o] = c;
                    else gc2[o] = c;                     // o < capacity: one entry per row
                }
                base += (uint32_t)__popcll(m[u]);
            }
        }
    }
    lds_barrier();
    const uint32_t nh = n_hit;
    if (nh > (uint32_t)kFinalLds) {                      // the radix passes then read one contiguous list
        for (uint32_t i = t; i < (uint32_t)kFinalLds; i += kRowThreads) gc2[i] = L.lc[i];
        __threadfence_block();                             // (only then: it waits for every store)
        __syncthreads();
    }
    zero_hist(hb);                                       // read above; the stores drain during the radix
    // every hit above bin T, and the need = want - above largest of bin T
    const uint32_t above = above_s, need = want > above ? want - above : 0u;
    if (nh <= (uint32_t)kFinalLds)
        radix_take_bins<kRowThreads>(L.lc, nh, T, in_t_s, true, need, want, out, &cursor, L.h, L.res);
    else
        radix_take_bins<kRowThreads>(gc2, nh, T, in_t_s, true, need, want, out, &cursor, L.h, L.res);
    __syncthreads();
    for (uint32_t i = want + t; i < (uint32_t)k; i += kRowThreads) out.put(i, -1);
}

// ---- many workgroups per sequence ------------------------------------------
template <bool POOL>
__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ scores, int64_t capacity,
                                                        const int32_t* __restrict__ n_visible, int k,
                                                        TopkWorkspace ws, SelectMap map) {
    __shared__ uint64_t cnd[kSelRows];
    __shared__ int32_t sel[kSelRows];
    __shared__ uint32_t n_sel, n_cnd;
    __shared__ int T_s;
    const int b = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63;
    constexpr int kPer = kSelRows / kSelThreads;
    // the slice's scores are loaded before the threshold search, so both latencies overlap
    const int64_t nvis = visible_of(n_visible, b, capacity);
    const int64_t r0 = (int64_t)blockIdx.x * kSelRows;
    const float* sc = scores + b * capacity;
    const auto pmap = pos_map<POOL>(map, b);
    const int32_t* __restrict__ cb = POOL ? map.cand + b * capacity : nullptr;
    float v[kPer];
    int32_t cv[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t s = r0 + i * kSelThreads + t;
        v[i] = (s < nvis) ? sc[s] : 0.0f;
        if constexpr (POOL) cv[i] = (s < nvis) ? cb[s] : 0;
        else cv[i] = 0;
    }
    if (t < 64) {
        const DigitResult r = hist_find(ws.hist + (int64_t)b * kHistWordsHost, (uint32_t)k);
        if (t == 0) {
            T_s = r.found ? r.digit : -1;
            n_sel = 0;
            n_cnd = 0;
        }
    }
    lds_barrier();
    const int T = T_s;
    uint32_t key[kPer];
    uint64_t mt[kPer], mc[kPer];
    uint32_t nt = 0, nc = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int64_t s = r0 + i * kSelThreads + t;
        bool take, maybe;
        classify(v[i], s < nvis, T, &key[i], &take, &maybe);
        mt[i] = __ballot(take);
        mc[i] = __ballot(maybe);
        nt += (uint32_t)__popcll(mt[i]);
        nc += (uint32_t)__popcll(mc[i]);
    }
    if (nt | nc) {                                       // one LDS reservation per wave and list
        uint32_t bt = 0, bc = 0;
        if (lane == 0) {
            if (nt) bt = atomicAdd(&n_sel, nt);
            if (nc) bc = atomicAdd(&n_cnd, nc);
        }
        bt = __shfl(bt, 0, 64);
        bc = __shfl(bc, 0, 64);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int64_t s = r0 + i * kSelThreads + t;
            if ((mt[i] >> lane) & 1u) sel[bt + lanes_below(mt[i])] = pmap(s, cv[i]);
            if ((mc[i] >> lane) & 1u)
                cnd[bc + lanes_below(mc[i])] = ((uint64_t)key[i] << 32) | (uint64_t)(~(uint32_t)pmap(s, cv[i]));
            bt += (uint32_t)__popcll(mt[i]);
            bc += (uint32_t)__popcll(mc[i]);
        }
    }
    lds_barrier();
    // this workgroup's share of zeroing the fine histogram for the next call: every
    // workgroup of the sequence finds the same threshold, so only the 64 fine bins of
    // the threshold's coarse bin (which the others may still be reading, and which
    // k_select_final clears) are skipped. (Issued after the classification: a load
    // waited for behind a store waits for that store too.)
    {
        uint32_t* fine0 = hist_fine(ws.hist + (int64_t)b * kHistWordsHost, 0);
        constexpr int kFineWords = kHistCopies * kHistBins;
        const int per = (kFineWords / 4 + gridDim.x - 1) / gridDim.x;   // u32x4 per workgroup
        const int cb = T >= 0 ? T / kFinePerCoarse : -1;
        for (int i = blockIdx.x * per + t; i < (int)(blockIdx.x + 1) * per && i < kFineWords / 4; i += kSelThreads)
            if (((4 * i) % kHistBins) / kFinePerCoarse != cb)
                reinterpret_cast<u32x4*>(fine0)[i] = u32x4{0u, 0u, 0u, 0u};
    }
    // the workgroup's own slots: counts, then its lists at r0 (at most kSelRows rows each)
    if (t == 0) {
        uint32_t* cnt = ws.counts + ((int64_t)b * gridDim.x + blockIdx.x) * 2;
        cnt[0] = n_sel;
        cnt[1] = n_cnd;
    }
    int32_t* gsel = ws.sel + b * capacity + r0;
    uint64_t* gcnd = ws.cand + b * capacity + r0;
    for (uint32_t i = t; i < n_sel; i += kSelThreads) gsel[i] = sel[i];
    for (uint32_t i = t; i < n_cnd; i += kSelThreads) gcnd[i] = cnd[i];
}

// Inclusive prefix sum over the kSelThreads threads of the workgroup (all call it).
__device__ uint32_t block_incl_scan(uint32_t v, uint32_t* total) {
    __shared__ uint32_t wsum[kSelThreads / 64];
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    uint32_t incl = wave_incl_scan(v);
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    uint32_t off = 0, tot = 0;
    for (int i = 0; i < kSelThreads / 64; ++i) {
        off += (i < wv) ? wsum[i] : 0u;
        tot += wsum[i];
    }
    __syncthreads();
    *total = tot;
    return incl + off;
}

// One workgroup per sequence, after every k_select workgroup of it: prefix-sum the
// counts, gather the selected positions into the output and the candidates into
// one list, radix-select among the candidates, pad with -1.
template <bool EXPAND>
__global__ __launch_bounds__(kSelThreads) void k_select_final(const int32_t* __restrict__ n_visible, int k,
                                                              int64_t capacity, int groups, TopkWorkspace ws,
                                                              int32_t* __restrict__ out_idx, SelectMap map) {
    __shared__ FinalLds L;
    __shared__ uint32_t cursor;
    __shared__ uint32_t ex_s[kSelThreads], ex_c[kSelThreads], cnt_s[kSelThreads], cnt_c[kSelThreads];
    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63;
    const int64_t nvis = visible_of(n_visible, b, capacity);
    const uint32_t want = (uint32_t)((nvis < k) ? nvis : k);
    const auto out = out_row<EXPAND>(out_idx, b, k, map);
    uint64_t* gc2 = ws.cand2 + b * capacity;

    uint32_t nsel = 0, ncand = 0;
    constexpr int kGU = 16;
    const int wv = t >> 6;
    for (int g0 = 0; g0 < groups; g0 += kSelThreads) {
        const int gi = g0 + t;
        const int nbatch = (groups - g0 < kSelThreads) ? groups - g0 : kSelThreads;
        const int32_t* __restrict__ gsel = ws.sel + b * capacity + (int64_t)g0 * kSelRows;
        const uint64_t* __restrict__ gcnd = ws.cand + b * capacity + (int64_t)g0 * kSelRows;
        // the first 64 entries of 16 workgroups' lists per wave are loaded together with the
        // counts (whatever the counts turn out to be: the slots exist, stale entries are dropped)
        // the counts first: loads return in order, and the prefix sums need only them
        uint32_t cs = 0, cc = 0;
        if (gi < groups) {
            const u32x2 cnt = *reinterpret_cast<const u32x2*>(ws.counts + ((int64_t)b * groups + gi) * 2);
            cs = cnt.x;
            cc = cnt.y;
        }
        int32_t vs[kGU];
        uint64_t vc[kGU];
        const int64_t room = capacity - (int64_t)g0 * kSelRows;   // entries left in this batch's slots
#pragma unroll
        for (int u = 0; u < kGU; ++u) {
            const int j = wv + 4 * u;
            const int64_t off = (int64_t)j * kSelRows + lane;
            const bool ok = j < nbatch && off < room;
            vs[u] = ok ? gsel[off] : 0;
            vc[u] = ok ? gcnd[off] : 0ull;
        }
        uint32_t ts, tc;
        const uint32_t is = block_incl_scan(cs, &ts);
        const uint32_t ic = block_incl_scan(cc, &tc);
        ex_s[t] = is - cs;
        ex_c[t] = ic - cc;
        cnt_s[t] = cs;
        cnt_c[t] = cc;
        __syncthreads();
        // wave w places the lists of workgroups w, w + 4, ..: the first 64 entries of
        // workgroups w .. w + 60 were loaded above, later rounds load theirs here
        for (int jb = wv; jb < nbatch; jb += 4 * kGU) {
            if (jb != wv) {
#pragma unroll
                for (int u = 0; u < kGU; ++u) {
                    const int j = jb + 4 * u;
                    const uint32_t ns = (j < nbatch) ? cnt_s[j] : 0u, nc = (j < nbatch) ? cnt_c[j] : 0u;
                    vs[u] = ((uint32_t)lane < ns) ? gsel[(int64_t)j * kSelRows + lane] : 0;
                    vc[u] = ((uint32_t)lane < nc) ? gcnd[(int64_t)j * kSelRows + lane] : 0ull;
                }
            }
#pragma unroll
            for (int u = 0; u < kGU; ++u) {
                const int j = jb + 4 * u;
                if (j >= nbatch) break;
                if ((uint32_t)lane < cnt_s[j]) {
                    const uint32_t o = nsel + ex_s[j] + lane;
                    if (o < (uint32_t)k) out.put(o, vs[u]);
                }
                if ((uint32_t)lane < cnt_c[j]) {
                    const uint32_t o = ncand + ex_c[j] + lane;
                    if (o < (uint32_t)kFinalLds) L.lc[o] = vc[u];
                    else gc2[o] = vc[u];          // o < capacity: every row is in at most one list
                }
            }
        }
        // entries past the first 64 of a workgroup's list (concentrated selections)
        const bool long_lists = __syncthreads_or(cs > 64u || cc > 64u);
        for (int j = wv; long_lists && j < nbatch; j += 4) {
            const uint32_t ns = cnt_s[j], nc = cnt_c[j];
            for (uint32_t i0 = 64; i0 < ns; i0 += 64 * 8) {
                int32_t vv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t i = i0 + 64 * u + lane;
                    vv[u] = (i < ns) ? gsel[(int64_t)j * kSelRows + i] : 0;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t i = i0 + 64 * u + lane, o = nsel + ex_s[j] + i;
                    if (i < ns && o < (uint32_t)k) out.put(o, vv[u]);
                }
            }
            for (uint32_t i0 = 64; i0 < nc; i0 += 64 * 8) {
                uint64_t vv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t i = i0 + 64 * u + lane;
                    vv[u] = (i < nc) ? gcnd[(int64_t)j * kSelRows + i] : 0ull;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const uint32_t i = i0 + 64 * u + lane, o = ncand + ex_c[j] + i;
                    if (i >= nc) continue;
                    if (o < (uint32_t)kFinalLds) L.lc[o] = vv[u];
                    else gc2[o] = vv[u];
                }
            }
        }
        nsel += ts;
        ncand += tc;
        __syncthreads();
    }
    if (ncand > (uint32_t)kFinalLds)                     // the radix passes then read one contiguous list
        for (uint32_t i = t; i < (uint32_t)kFinalLds; i += kSelThreads) gc2[i] = L.lc[i];
    __threadfence_block();
    if (t == 0) cursor = nsel;
    for (int i = t; i < kMaxDigitBins; i += kSelThreads) L.h[0][i] = 0u;
    __syncthreads();
    const uint32_t need = (want > nsel) ? want - nsel : 0u;
    zero_hist_rest(ws.hist + (int64_t)b * kHistWordsHost, (uint32_t)k,
                   threadIdx.x < 64 ? coarse_sum_of_lane(ws.hist + (int64_t)b * kHistWordsHost) : 0u);   // the stores drain during the radix
    radix_take_any<kSelThreads>(L, gc2, ncand, need, want, out, &cursor);
    __syncthreads();
    for (uint32_t i = want + t; i < (uint32_t)k; i += kSelThreads) out.put(i, -1);
}

constexpr int kF2Threads = 1024;
constexpr int kF2Waves = kF2Threads / 64;
constexpr int kF2MaxGroups = 1024;
constexpr int kF2Spec = 8;                // workgroups per wave whose first 64 entries load early (flat final)
constexpr int kF2Flat = 4;                // rest entries per thread per batch
constexpr int kSpecGroups = kF2Waves * kF2Spec;
// The final for up to 16 SPEC select workgroups (SPEC = 4 or 8), where every list's
// first 64 entries are loaded speculatively: wave w places the lists of
// workgroups w, w + 16, .., w + 16 (SPEC - 1) (the counts are loaded first, and the
// prefix sums wait only for them); entries past the first 64 of a list, which
// the selections here rarely have, are placed afterwards, 64 at a time.
template <bool EXPAND, int SPEC>
__global__ __launch_bounds__(kF2Threads) void k_select_final2(const int32_t* __restrict__ n_visible, int k,
                                                              int64_t capacity, int groups, TopkWorkspace ws,
                                                              int32_t* __restrict__ out_idx, SelectMap map) {
    __shared__ FinalLds L;
    __shared__ uint32_t cursor;
    __shared__ uint32_t g_cnt[kF2MaxGroups][2], g_off[kF2MaxGroups][2];
    __shared__ uint32_t wtot[kF2Waves][2];
    __shared__ uint32_t has_rest;
    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t nvis = visible_of(n_visible, b, capacity);
    const uint32_t want = (uint32_t)((nvis < k) ? nvis : k);
    const auto out = out_row<EXPAND>(out_idx, b, k, map);
    uint64_t* gc2 = ws.cand2 + b * capacity;
    const int32_t* __restrict__ gsel = ws.sel + b * capacity;
    const uint64_t* __restrict__ gcnd = ws.cand + b * capacity;

    // every load unconditional, from a clamped in-bounds address, so that the waits
    // for the counts (issued first) do not cover the list loads behind them
    // wave 0 also loads the coarse histogram sums the zeroing needs at the end
    const uint32_t csum = (t < 64) ? coarse_sum_of_lane(ws.hist + (int64_t)b * kHistWordsHost) : 0u;
    const bool has_cnt = t < groups;
    const u32x2 c2 = *reinterpret_cast<const u32x2*>(ws.counts + ((int64_t)b * groups + (has_cnt ? t : 0)) * 2);
    int32_t vs[SPEC];
    uint64_t vc[SPEC];
#pragma unroll
    for (int u = 0; u < SPEC; ++u) {
        const int j = wv + kF2Waves * u;
        const int64_t off = (int64_t)j * kSelRows + lane;
        const bool ok = j < groups && off < capacity;
        vs[u] = gsel[ok ? off : 0];
        vc[u] = gcnd[ok ? off : 0];
        if (!ok) {
            vs[u] = 0;
            vc[u] = 0ull;
        }
    }
    const uint32_t cs = has_cnt ? c2.x : 0u, cc = has_cnt ? c2.y : 0u;
    // exclusive prefix sums of the counts over the workgroups
    const uint32_t is = wave_incl_scan(cs), ic = wave_incl_scan(cc);
    if (lane == 63) {
        wtot[wv][0] = is;
        wtot[wv][1] = ic;
    }
    if (t == 0) has_rest = groups > (kF2Waves * SPEC) ? 1u : 0u;
    lds_barrier();
    uint32_t bs = 0, bc = 0, nsel = 0, ncand = 0;
#pragma unroll
    for (int i = 0; i < kF2Waves; ++i) {
        const uint32_t s_ = wtot[i][0], c_ = wtot[i][1];
        if (i < wv) {
            bs += s_;
            bc += c_;
        }
        nsel += s_;
        ncand += c_;
    }
    if (t < groups) {
        g_off[t][0] = bs + is - cs;
        g_off[t][1] = bc + ic - cc;
        g_cnt[t][0] = cs;
        g_cnt[t][1] = cc;
        if (cs > 64u || cc > 64u) has_rest = 1u;
    }
    lds_barrier();
    // placement: entry i of workgroup j's lists goes to the output (selected) or to
    // the candidate list (LDS, then cand2 past kFinalLds)
    auto place_sel = [&](int j, uint32_t i, int32_t v) {
        const uint32_t o = g_off[j][0] + i;
        if (o < (uint32_t)k) out.put(o, v);
    };
    auto place_cnd = [&](int j, uint32_t i, uint64_t v) {
        const uint32_t o = g_off[j][1] + i;
        if (o < (uint32_t)kFinalLds) L.lc[o] = v;
        else gc2[o] = v;                                   // o < capacity: every row is in at most one list
    };
#pragma unroll
    for (int u = 0; u < SPEC; ++u) {
        const int j = wv + kF2Waves * u;
        if (j < groups) {
            if ((uint32_t)lane < g_cnt[j][0]) place_sel(j, lane, vs[u]);
            if ((uint32_t)lane < g_cnt[j][1]) place_cnd(j, lane, vc[u]);
        }
    }
    // the rest: workgroups past the speculated ones, and entries past the first 64
    // (skipped as a whole when there is none: its loads, issued behind the output's
    // stores, would wait for them)
    if (has_rest) {
        for (int j = wv; j < groups; j += kF2Waves) {
            const uint32_t i0 = (j < wv + kF2Waves * SPEC) ? 64u : 0u;
            const uint32_t ns = g_cnt[j][0], nc = g_cnt[j][1];
            for (uint32_t i = i0 + lane; i < ns; i += 64) place_sel(j, i, gsel[(int64_t)j * kSelRows + i]);
            for (uint32_t i = i0 + lane; i < nc; i += 64) place_cnd(j, i, gcnd[(int64_t)j * kSelRows + i]);
        }
    }
    // the barriers below order LDS only (the output's stores need no ordering here);
    // a candidate list that overflows LDS is also read from global memory, so then
    // every store of it has landed first
    if (ncand > (uint32_t)kFinalLds) __threadfence_block();
    lds_barrier();
    if (ncand > (uint32_t)kFinalLds) {                   // the radix passes then read one contiguous list
        for (uint32_t i = t; i < (uint32_t)kFinalLds; i += kF2Threads) gc2[i] = L.lc[i];
        __threadfence_block();                             // (only then: it waits for every store)
    }
    if (t == 0) cursor = nsel;
    for (int i = t; i < kMaxDigitBins; i += kF2Threads) L.h[0][i] = 0u;
    lds_barrier();
    const uint32_t need = (want > nsel) ? want - nsel : 0u;
    zero_hist_rest(ws.hist + (int64_t)b * kHistWordsHost, (uint32_t)k, csum);   // the stores drain during the radix
    radix_take_any<kF2Threads>(L, gc2, ncand, need, want, out, &cursor);
    for (uint32_t i = want + t; i < (uint32_t)k; i += kF2Threads) out.put(i, -1);   // slots the take leaves alone
}


// The same for up to kF2MaxGroups select workgroups (and for selections of
// blocks, whose lists run longer), with 1024 threads. The counts are loaded first, then (from clamped in-bounds addresses, branch-free,
// so that the waits for the counts do not cover them) the first 64 entries of
// the lists of workgroups w, w + 16, w + 32, w + 48 by wave w, speculatively.
// Prefix sums of the counts (one DPP scan per wave, one LDS pass) give every
// workgroup's offsets in the output and in the candidate list, and prefix sums
// of what the speculative loads did not cover (entries past the first 64, and
// the lists of workgroups past the first 64) place "the rest" in one flat
// index space: rest entry r belongs to the last workgroup whose rest offset is
// <= r (a binary search in LDS). Each thread issues the loads of its rest
// entries before it stores anything (a load issued behind a store waits for
// that store: the vector memory counter counts both), so the rest costs one
// load latency however the entries spread over the workgroups.
template <bool EXPAND>
__global__ __launch_bounds__(kF2Threads) void k_select_final2_flat(const int32_t* __restrict__ n_visible, int k,
                                                              int64_t capacity, int groups, TopkWorkspace ws,
                                                              int32_t* __restrict__ out_idx, SelectMap map) {
    __shared__ FinalLds L;
    __shared__ uint32_t cursor;
    __shared__ uint32_t g_off[2][kF2MaxGroups], g_cnt[2][kF2MaxGroups], r_off[2][kF2MaxGroups];
    __shared__ uint32_t wtot[kF2Waves][4];
    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    const int64_t nvis = visible_of(n_visible, b, capacity);
    const uint32_t want = (uint32_t)((nvis < k) ? nvis : k);
    const auto out = out_row<EXPAND>(out_idx, b, k, map);
    uint64_t* gc2 = ws.cand2 + b * capacity;
    const int32_t* __restrict__ gsel = ws.sel + b * capacity;
    const uint64_t* __restrict__ gcnd = ws.cand + b * capacity;

    // wave 0 also loads the coarse histogram sums the zeroing needs at the end
    const uint32_t csum = (t < 64) ? coarse_sum_of_lane(ws.hist + (int64_t)b * kHistWordsHost) : 0u;
    const bool has_cnt = t < groups;
    const u32x2 c2 = *reinterpret_cast<const u32x2*>(ws.counts + ((int64_t)b * groups + (has_cnt ? t : 0)) * 2);
    int32_t vs[kF2Spec];
    uint64_t vc[kF2Spec];
#pragma unroll
    for (int u = 0; u < kF2Spec; ++u) {
        const int j = wv + kF2Waves * u;
        const int64_t off = (int64_t)j * kSelRows + lane;
        const bool ok = j < groups && off < capacity;
        vs[u] = gsel[ok ? off : 0];
        vc[u] = gcnd[ok ? off : 0];
        if (!ok) {
            vs[u] = 0;
            vc[u] = 0ull;
        }
    }
    const uint32_t cs = has_cnt ? c2.x : 0u, cc = has_cnt ? c2.y : 0u;
    const bool spec = t < kSpecGroups;
    const uint32_t rs = spec ? cs - min(cs, 64u) : cs, rc = spec ? cc - min(cc, 64u) : cc;
    // exclusive prefix sums over the workgroups: offsets, and offsets of the rest
    const uint32_t is = wave_incl_scan(cs), ic = wave_incl_scan(cc);
    const uint32_t irs = wave_incl_scan(rs), irc = wave_incl_scan(rc);
    if (lane == 63) {
        wtot[wv][0] = is;
        wtot[wv][1] = ic;
        wtot[wv][2] = irs;
        wtot[wv][3] = irc;
    }
    lds_barrier();
    uint32_t bs = 0, bc = 0, brs = 0, brc = 0, nsel = 0, ncand = 0, nrs = 0, nrc = 0;
#pragma unroll
    for (int i = 0; i < kF2Waves; ++i) {
        const uint32_t s_ = wtot[i][0], c_ = wtot[i][1], rs_ = wtot[i][2], rc_ = wtot[i][3];
        if (i < wv) {
            bs += s_;
            bc += c_;
            brs += rs_;
            brc += rc_;
        }
        nsel += s_;
        ncand += c_;
        nrs += rs_;
        nrc += rc_;
    }
    if (t < groups) {
        g_off[0][t] = bs + is - cs;
        g_off[1][t] = bc + ic - cc;
        g_cnt[0][t] = cs;
        g_cnt[1][t] = cc;
        r_off[0][t] = brs + irs - rs;
        r_off[1][t] = brc + irc - rc;
    }
    lds_barrier();
    // placement: entry i of workgroup j's lists goes to the output (selected) or to
    // the candidate list (LDS, then cand2 past kFinalLds)
    auto place = [&](int w, int j, uint32_t i, uint64_t v) {
        const uint32_t o = g_off[w][j] + i;
        if (w == 0) {
            if (o < (uint32_t)k) out.put(o, (int32_t)(uint32_t)v);
        } else {
            if (o < (uint32_t)kFinalLds) L.lc[o] = v;
            else gc2[o] = v;                               // o < capacity: every row is in at most one list
        }
    };
    // the workgroup holding rest entry r of list w: the last one whose rest offset is <= r
    auto owner = [&](int w, uint32_t r) -> int {
        int lo = 0, hi = groups - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (r_off[w][mid] <= r) lo = mid;
            else hi = mid - 1;
        }
        return lo;
    };
    const uint32_t n_rest = nrs + nrc;
    bool spec_placed = false;
    for (uint32_t base = 0; base == 0 || base < n_rest; base += kF2Flat * kF2Threads) {
        uint64_t rv[kF2Flat];
        int rj[kF2Flat];
        uint32_t ri[kF2Flat];
#pragma unroll
        for (int u = 0; u < kF2Flat; ++u) {
            const uint32_t r = base + u * kF2Threads + t;
            rj[u] = -1;
            if (r < nrs) {
                const int j = owner(0, r);
                const uint32_t i = (j < kSpecGroups ? 64u : 0u) + (r - r_off[0][j]);
                rj[u] = j;
                ri[u] = i;
                rv[u] = (uint64_t)(uint32_t)gsel[(int64_t)j * kSelRows + i];
            } else if (r < n_rest) {
                const uint32_t rr = r - nrs;
                const int j = owner(1, rr);
                const uint32_t i = (j < kSpecGroups ? 64u : 0u) + (rr - r_off[1][j]);
                rj[u] = j + kF2MaxGroups;                  // (list 1)
                ri[u] = i;
                rv[u] = gcnd[(int64_t)j * kSelRows + i];
            }
        }
        if (!spec_placed) {                                // the speculated entries, behind the first rest loads
            spec_placed = true;
#pragma unroll
            for (int u = 0; u < kF2Spec; ++u) {
                const int j = wv + kF2Waves * u;
                if (j < groups) {
                    if ((uint32_t)lane < g_cnt[0][j]) place(0, j, lane, (uint64_t)(uint32_t)vs[u]);
                    if ((uint32_t)lane < g_cnt[1][j]) place(1, j, lane, vc[u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kF2Flat; ++u) {
            if (rj[u] >= kF2MaxGroups) place(1, rj[u] - kF2MaxGroups, ri[u], rv[u]);
            else if (rj[u] >= 0) place(0, rj[u], ri[u], rv[u]);
        }
    }
    lds_barrier();
    if (ncand > (uint32_t)kFinalLds) {                   // the radix passes then read one contiguous list
        for (uint32_t i = t; i < (uint32_t)kFinalLds; i += kF2Threads) gc2[i] = L.lc[i];
        __threadfence_block();                             // (only then: it waits for every store)
        __syncthreads();
    }
    if (t == 0) cursor = nsel;
    for (int i = t; i < kMaxDigitBins; i += kF2Threads) L.h[0][i] = 0u;
    lds_barrier();
    const uint32_t need = (want > nsel) ? want - nsel : 0u;
    zero_hist_rest(ws.hist + (int64_t)b * kHistWordsHost, (uint32_t)k, csum);   // the stores drain during the radix
    radix_take_any<kF2Threads>(L, gc2, ncand, need, want, out, &cursor);
    for (uint32_t i = want + t; i < (uint32_t)k; i += kF2Threads) out.put(i, -1);   // slots the take leaves alone
}

}  // namespace

hipError_t launch_select_lists(const float* scores, int64_t capacity, const int32_t* n_visible, int B, int k,
                               const TopkWorkspace& ws, hipStream_t stream, int* groups) {
    *groups = 0;
    if (B == 0 || k == 0) return hipSuccess;
    bool row = capacity < kFoldManyMin;
    if (const int64_t path = option(OPT_TOPK_PATH)) row = path == 1;
    const int64_t nx = (capacity + kSelRows - 1) / kSelRows;
    if (row || nx < 1 || nx > kFusedSelectGroups) return hipSuccess;
    const ProfSlot p = prof_slot(PROF_SELECT);
    const hipError_t e = launch_kernel(k_select<false>, dim3((unsigned)nx, B), dim3(kSelThreads), 0, stream, p.start,
                                       p.stop, scores, capacity, n_visible, k, ws, SelectMap{});
    if (e == hipSuccess) *groups = (int)nx;
    return e;
}

// Options topk_path (1 row, 2 multi) and topk_final (1: the 256-thread final) force a path.
hipError_t launch_select(const float* scores, int64_t capacity, const int32_t* n_visible, int B, int k,
                         const TopkWorkspace& ws, int32_t* out_idx, hipStream_t stream, const SelectMap& map) {
    if (B == 0 || k == 0) return hipSuccess;
    const bool pool = map.cand != nullptr, expand = map.expand != 1;
    bool row = capacity <= kRowPathMax;
    if (const int64_t path = option(OPT_TOPK_PATH)) row = path == 1;
    const ProfSlot p = prof_slot(PROF_SELECT);      // spans both kernels of the two-kernel path
    if (row) {
        auto kr = pool ? (expand ? k_topk_row<true, true> : k_topk_row<true, false>)
                       : (expand ? k_topk_row<false, true> : k_topk_row<false, false>);
        return launch_kernel(kr, dim3(B), dim3(kRowThreads), 0, stream, p.start, p.stop, scores, capacity,
                             n_visible, k, ws, out_idx, map);
    }
    const unsigned nx = (unsigned)((capacity + kSelRows - 1) / kSelRows);
    if (nx > 0) {
        const hipError_t e = launch_kernel(pool ? k_select<true> : k_select<false>, dim3(nx, B),
                                           dim3(kSelThreads), 0, stream, p.start, nullptr,
                                           scores, capacity, n_visible, k, ws, map);
        if (e != hipSuccess) return e;
    }
    if (nx <= (unsigned)kF2MaxGroups && option(OPT_TOPK_FINAL) == 0)
        return launch_kernel(expand ? k_select_final2_flat<true>
                                    : (nx > (unsigned)kSpecGroups ? k_select_final2_flat<false>
                                       : nx > (unsigned)(kF2Waves * 4) ? k_select_final2<false, 8>
                                                                       : k_select_final2<false, 4>),
                             dim3(B), dim3(kF2Threads), 0, stream, nx > 0 ? nullptr : p.start,
                             p.stop, n_visible, k, capacity, (int)nx, ws, out_idx, map);
    return launch_kernel(expand ? k_select_final<true> : k_select_final<false>, dim3(B), dim3(kSelThreads), 0,
                         stream, nx > 0 ? nullptr : p.start, p.stop, n_visible, k, capacity, (int)nx, ws, out_idx,
                         map);
}

}  // namespace mla
