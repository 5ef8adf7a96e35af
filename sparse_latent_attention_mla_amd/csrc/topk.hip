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
//      key << 32 | ~position), then reserves space for both lists with one
//      global atomic each and copies them out;
//   3. k_select_final (one workgroup per sequence) radix-selects the missing
//      count among the candidates (the 52 free bits of the 64-bit composite,
//      most significant digit first, so the smaller position wins a tie) and
//      pads with -1.
// Output positions form an unordered set.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kSelThreads = 256;
constexpr int kSelRows = 2048;            // rows per k_select workgroup
constexpr int kFinalThreads = 1024;
constexpr int kFinalLds = 7168;           // candidates kept in LDS (56 KB)

__global__ void k_topk_clear(TopkWorkspace ws, int B) {
    const int b = blockIdx.x;
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) ws.hist[(int64_t)b * kHistBins + i] = 0u;
    if (threadIdx.x < 4) ws.counters[b * 4 + threadIdx.x] = 0u;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    return v;
}

// Suffix search over `nb` (<= 4 * 64) counts held one per thread, thread t holding
// the count of rank t in DESCENDING order (t = 0 is the largest bin).  Finds the
// rank r with  sum_{t<r} c_t < need <= sum_{t<=r} c_t  and the sum before it.
// All threads of the workgroup must call it; threads >= nb pass c = 0.
// Result in *rank (-1 if the total is below need) and *before.
__device__ void find_rank(uint32_t c, uint32_t need, int* rank, uint32_t* before, uint32_t* wsum) {
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    uint32_t incl = (t < 256) ? wave_incl_scan(c) : 0u;
    if (t < 256 && lane == 63) wsum[wv] = incl;
    if (t == 0) *rank = -1;
    __syncthreads();
    if (t < 256) {
        uint32_t off = 0;
        for (int i = 0; i < wv; ++i) off += wsum[i];
        incl += off;
        const uint32_t excl = incl - c;
        if (excl < need && incl >= need) { *rank = t; *before = excl; }
    }
    __syncthreads();
}

// Threshold bin of sequence b: the bin T holding the k-th largest key and the
// number of keys above it.  T = -1 when every visible row fits in k.
__device__ void find_threshold(const uint32_t* __restrict__ hist, int k, int* T_out, uint32_t* above_out) {
    __shared__ uint32_t wsum[4];
    __shared__ int rank_s;
    __shared__ uint32_t before_s;
    __shared__ int T_s;
    __shared__ uint32_t above_s;
    const int t = threadIdx.x;                       // kSelThreads == 256
    constexpr int per = kHistBins / kSelThreads;     // 16 bins per thread, top bins first
    const int hi = kHistBins - 1 - t * per;
    uint32_t cnt[per];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < per; ++i) { cnt[i] = hist[hi - i]; sum += cnt[i]; }
    find_rank(sum, (uint32_t)k, &rank_s, &before_s, wsum);
    if (t == 0) { T_s = -1; above_s = 0; }
    __syncthreads();
    if (t == rank_s) {
        uint32_t run = before_s;
#pragma unroll
        for (int i = 0; i < per; ++i) {
            if (run + cnt[i] >= (uint32_t)k) { T_s = hi - i; above_s = run; break; }
            run += cnt[i];
        }
    }
    __syncthreads();
    *T_out = T_s;
    *above_out = above_s;
}

__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ scores, int64_t capacity,
                                                        const int32_t* __restrict__ n_visible, int k,
                                                        TopkWorkspace ws, int32_t* __restrict__ out_idx) {
    __shared__ int32_t sel[kSelRows];
    __shared__ uint64_t cnd[kSelRows];
    __shared__ uint32_t n_sel, n_cnd, base_sel, base_cnd;
    const int b = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63;
    int T;
    uint32_t above;
    find_threshold(ws.hist + (int64_t)b * kHistBins, k, &T, &above);
    const int64_t nvis = clamp_visible(n_visible[b], capacity);
    const int64_t r0 = (int64_t)blockIdx.x * kSelRows;
    if (t == 0) { n_sel = 0; n_cnd = 0; }
    __syncthreads();
    const float* sc = scores + b * capacity;
    for (int i = 0; i < kSelRows / kSelThreads; ++i) {
        const int64_t s = r0 + i * kSelThreads + t;
        const bool in = s < nvis;
        uint32_t key = 0, bin = 0;
        if (in) {
            key = score_key(sc[s]);
            bin = key >> (32 - kHistBits);
        }
        const bool take = in && (T < 0 || (int)bin > T);
        const bool maybe = in && T >= 0 && (int)bin == T;
        const uint64_t mt = __ballot(take), mc = __ballot(maybe);
        uint32_t bt = 0, bc = 0;
        if (lane == 0) {
            if (mt) bt = atomicAdd(&n_sel, (uint32_t)__popcll(mt));
            if (mc) bc = atomicAdd(&n_cnd, (uint32_t)__popcll(mc));
        }
        bt = __shfl(bt, 0, 64);
        bc = __shfl(bc, 0, 64);
        if (take) sel[bt + lanes_below(mt)] = (int32_t)s;
        if (maybe) cnd[bc + lanes_below(mc)] = ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)s);
    }
    __syncthreads();
    if (t == 0) {
        base_sel = n_sel ? atomicAdd(&ws.counters[b * 4 + 0], n_sel) : 0u;
        base_cnd = n_cnd ? atomicAdd(&ws.counters[b * 4 + 1], n_cnd) : 0u;
    }
    __syncthreads();
    int32_t* out = out_idx + (int64_t)b * k;
    for (uint32_t i = t; i < n_sel; i += kSelThreads)
        if (base_sel + i < (uint32_t)k) out[base_sel + i] = sel[i];
    uint64_t* cand = ws.cand + b * capacity;
    for (uint32_t i = t; i < n_cnd; i += kSelThreads)
        if (base_cnd + i < (uint64_t)capacity) cand[base_cnd + i] = cnd[i];
}

// One workgroup per sequence.
__global__ __launch_bounds__(kFinalThreads) void k_select_final(const int32_t* __restrict__ n_visible, int k,
                                                               int64_t capacity, TopkWorkspace ws,
                                                               int32_t* __restrict__ out_idx) {
    __shared__ uint64_t lc[kFinalLds];
    __shared__ uint32_t h256[256];
    __shared__ uint32_t wsum[4];
    __shared__ int rank_s;
    __shared__ uint32_t before_s;
    __shared__ uint32_t cursor;
    const int b = blockIdx.x;
    const int t = threadIdx.x, lane = t & 63;
    const int64_t nvis = clamp_visible(n_visible[b], capacity);
    const uint32_t want = (uint32_t)((nvis < k) ? nvis : k);
    const uint32_t nsel = ws.counters[b * 4 + 0];
    uint32_t ncand = ws.counters[b * 4 + 1];
    if (ncand > (uint64_t)capacity) ncand = (uint32_t)capacity;
    int32_t* out = out_idx + (int64_t)b * k;
    const uint64_t* gcand = ws.cand + b * capacity;
    const uint32_t need = (want > nsel) ? want - nsel : 0u;

    const bool in_lds = ncand <= (uint32_t)kFinalLds;
    if (in_lds)
        for (uint32_t i = t; i < ncand; i += kFinalThreads) lc[i] = gcand[i];
    if (t == 0) cursor = nsel;
    __syncthreads();
    const uint64_t* c = in_lds ? lc : gcand;

    // the need-th largest 64-bit composite; bits 63..52 (the bin) are equal
    const bool radix = need > 0 && need < ncand;
    constexpr uint64_t kBinBits = 0xFFFull << 52;    // shared by every candidate (the threshold bin)
    uint64_t prefix = radix ? (c[0] & kBinBits) : 0ull, mask = kBinBits;
    uint32_t rem = need;
    if (radix) {
        // digit windows 44..51, 36..43, .., 4..11, then 0..7 (bits 4..7 already fixed);
        // computed, not tabled: a constant table would be read from the code object
        for (int p = 0; p < 7; ++p) {
            const int shift = (p < 6) ? 44 - 8 * p : 0;
            if (t < 256) h256[t] = 0u;
            __syncthreads();
            for (uint32_t i = t; i < ncand; i += kFinalThreads) {
                const uint64_t v = c[i];
                if ((v & mask) == prefix) atomicAdd(&h256[(v >> shift) & 255u], 1u);
            }
            __syncthreads();
            // descending digit order: thread t holds digit 255 - t
            find_rank(t < 256 ? h256[255 - t] : 0u, rem, &rank_s, &before_s, wsum);
            const int d = 255 - (rank_s < 0 ? 0 : rank_s);
            prefix |= (uint64_t)d << shift;
            mask |= (uint64_t)255u << shift;
            rem -= before_s;
        }
    }
    // composites are unique (positions are): "v >= the need-th largest" is exactly `need` of them
    if (need > 0) {
        const uint32_t n_iter = (ncand + kFinalThreads - 1) / kFinalThreads;
        for (uint32_t it = 0; it < n_iter; ++it) {
            const uint32_t i = it * kFinalThreads + t;
            bool take = false;
            int32_t pos = 0;
            if (i < ncand) {
                const uint64_t v = c[i];
                take = !radix || v >= prefix;
                pos = (int32_t)(~(uint32_t)(v & 0xFFFFFFFFull));
            }
            const uint64_t m = __ballot(take);
            uint32_t base = 0;
            if (lane == 0 && m) base = atomicAdd(&cursor, (uint32_t)__popcll(m));
            base = __shfl(base, 0, 64);
            if (take) {
                const uint32_t o = base + lanes_below(m);
                if (o < want) out[o] = pos;
            }
        }
    }
    __syncthreads();
    for (uint32_t i = want + t; i < (uint32_t)k; i += kFinalThreads) out[i] = -1;
}

}  // namespace

hipError_t launch_topk_clear(const TopkWorkspace& ws, int B, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    hipLaunchKernelGGL(k_topk_clear, dim3(B), dim3(256), 0, stream, ws, B);
    return hipGetLastError();
}

hipError_t launch_select(const float* scores, int64_t capacity, const int32_t* n_visible, int B, int k,
                         const TopkWorkspace& ws, int32_t* out_idx, hipStream_t stream) {
    if (B == 0 || k == 0) return hipSuccess;
    const unsigned nx = (unsigned)((capacity + kSelRows - 1) / kSelRows);
    if (nx > 0) {
        hipLaunchKernelGGL(k_select, dim3(nx, B), dim3(kSelThreads), 0, stream, scores, capacity, n_visible, k,
                           ws, out_idx);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_select_final, dim3(B), dim3(kFinalThreads), 0, stream, n_visible, k, capacity, ws,
                       out_idx);
    return hipGetLastError();
}

}  // namespace mla
