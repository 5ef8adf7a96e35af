// topk.hip -- exact top-k over the indexer scores.
//
// Selection ([P1] "DeepSeek's Attention and KV Cache - From MLA to CSA2",
// "DeepSeek-V3.2", eq. 2; [P2] "From MLA to DSA to HCA/CSA", Part 1): the k
// visible rows of largest score, ties at the k-th score going to the smaller
// position; slots past min(k, n_visible) hold -1 ([P2] "CSA: two changes to
// HCA").  Radix selection on order-preserving score keys:
//   1. the scan kernel has built a histogram of the top kHistBits key bits;
//   2. k_select (many workgroups per sequence) finds the bin holding the k-th
//      largest key, emits every row of a higher bin straight into the output
//      and compacts the rows of that bin as 64-bit candidates
//      (key << 32 | ~position);
//   3. k_select_final (one workgroup per sequence) radix-selects the missing
//      count among the candidates (usually ~1% of the rows) and pads with -1.
// Output positions form an unordered set.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kSelThreads = 256;
constexpr int kSelRowsPerBlock = 8192;
constexpr int kFinalThreads = 1024;
constexpr int kFinalLds = 8192;          // candidates kept in LDS (64 KB)

__global__ void k_topk_clear(TopkWorkspace ws, int B) {
    const int b = blockIdx.x;
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) ws.hist[(int64_t)b * kHistBins + i] = 0u;
    if (threadIdx.x < 4) ws.counters[b * 4 + threadIdx.x] = 0u;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Append `flag` lanes' values at a global cursor, one atomic per wave.
template <typename T>
__device__ __forceinline__ void wave_append(bool flag, T value, uint32_t* cursor, T* dst, uint32_t limit) {
    const uint64_t mask = __ballot(flag);
    if (!mask) return;
    const uint32_t n = (uint32_t)__popcll(mask);
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((long long)mask) - 1;
    uint32_t base = 0;
    if (lane == leader) base = atomicAdd(cursor, n);
    base = __shfl(base, leader, 64);
    if (flag) {
        const uint32_t pos = base + lanes_below(mask);
        if (pos < limit) dst[pos] = value;
    }
}

// Threshold bin of sequence b: the bin T holding the k-th largest key, and the
// number of keys in bins above T.  T = -1 when every visible row fits in k.
__device__ void find_threshold(const uint32_t* __restrict__ hist, int k, int* T_out, uint32_t* above_out) {
    __shared__ uint32_t part[kSelThreads];
    __shared__ int T_s;
    __shared__ uint32_t above_s;
    const int t = threadIdx.x;
    constexpr int per = kHistBins / kSelThreads;          // 16 bins per thread, top bins first
    const int hi = kHistBins - 1 - t * per;
    uint32_t sum = 0;
    for (int i = 0; i < per; ++i) sum += hist[hi - i];
    part[t] = sum;
    if (t == 0) { T_s = -1; above_s = 0; }
    __syncthreads();
    // inclusive scan over threads (top bins first), Hillis-Steele in LDS
    for (int o = 1; o < kSelThreads; o <<= 1) {
        const uint32_t v = (t >= o) ? part[t - o] : 0u;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    const uint32_t incl = part[t], excl = incl - sum;
    if (excl < (uint32_t)k && incl >= (uint32_t)k) {
        uint32_t run = excl;
        for (int i = 0; i < per; ++i) {
            const uint32_t c = hist[hi - i];
            if (run + c >= (uint32_t)k) { T_s = hi - i; above_s = run; break; }
            run += c;
        }
    }
    __syncthreads();
    *T_out = T_s;
    *above_out = above_s;
}

__global__ __launch_bounds__(kSelThreads) void k_select(const float* __restrict__ scores, int64_t capacity,
                                                        const int32_t* __restrict__ n_visible, int k,
                                                        TopkWorkspace ws, int32_t* __restrict__ out_idx) {
    const int b = blockIdx.y;
    int T;
    uint32_t above;
    find_threshold(ws.hist + (int64_t)b * kHistBins, k, &T, &above);
    const int64_t nvis = clamp_visible(n_visible[b], capacity);
    const int64_t r0 = (int64_t)blockIdx.x * kSelRowsPerBlock;
    const float* sc = scores + b * capacity;
    uint32_t* ctr = ws.counters + b * 4;
    int32_t* out = out_idx + (int64_t)b * k;
    uint64_t* cand = ws.cand + b * capacity;
    // every lane of a wave runs the same number of iterations (wave_append is wave-wide)
    for (int64_t base = r0; base < r0 + kSelRowsPerBlock && base < nvis; base += kSelThreads) {
        const int64_t s = base + threadIdx.x;
        const bool in = s < nvis && s < r0 + kSelRowsPerBlock;
        uint32_t key = 0, bin = 0;
        if (in) {
            key = score_key(sc[s]);
            bin = key >> (32 - kHistBits);
        }
        const bool take = in && (T < 0 || (int)bin > T);
        const bool maybe = in && T >= 0 && (int)bin == T;
        wave_append<int32_t>(take, (int32_t)s, &ctr[0], out, (uint32_t)k);
        wave_append<uint64_t>(maybe, ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)s), &ctr[1], cand,
                              (uint32_t)capacity);
    }
}

// One workgroup per sequence.
__global__ __launch_bounds__(kFinalThreads) void k_select_final(const int32_t* __restrict__ n_visible, int k,
                                                               int64_t capacity, TopkWorkspace ws,
                                                               int32_t* __restrict__ out_idx) {
    __shared__ uint64_t lc[kFinalLds];
    __shared__ uint32_t h256[256];
    __shared__ uint64_t prefix_s;
    __shared__ uint32_t need_s;
    __shared__ uint32_t cursor;
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int64_t nvis = clamp_visible(n_visible[b], capacity);
    const uint32_t want = (uint32_t)((nvis < k) ? nvis : k);
    const uint32_t nsel = ws.counters[b * 4 + 0];
    const uint32_t ncand = ws.counters[b * 4 + 1];
    int32_t* out = out_idx + (int64_t)b * k;
    const uint64_t* gcand = ws.cand + b * capacity;
    const uint32_t need = (want > nsel) ? want - nsel : 0u;

    const bool in_lds = ncand <= (uint32_t)kFinalLds;
    if (in_lds)
        for (uint32_t i = t; i < ncand; i += kFinalThreads) lc[i] = gcand[i];
    if (t == 0) { prefix_s = 0; need_s = need; cursor = nsel; }
    __syncthreads();
    const uint64_t* c = in_lds ? lc : gcand;

    if (need > 0 && need < ncand) {
        // most-significant-digit radix select of the need-th largest 64-bit key
        uint64_t mask = 0;
        for (int shift = 56; shift >= 0; shift -= 8) {
            for (int i = t; i < 256; i += kFinalThreads) h256[i] = 0u;
            __syncthreads();
            const uint64_t prefix = prefix_s;
            for (uint32_t i = t; i < ncand; i += kFinalThreads) {
                const uint64_t v = c[i];
                if ((v & mask) == prefix) atomicAdd(&h256[(v >> shift) & 255u], 1u);
            }
            __syncthreads();
            if (t == 0) {
                uint32_t rem = need_s, run = 0;
                for (int d = 255; d >= 0; --d) {
                    if (run + h256[d] >= rem) {
                        prefix_s = prefix | ((uint64_t)d << shift);
                        need_s = rem - run;
                        break;
                    }
                    run += h256[d];
                }
            }
            mask |= (uint64_t)255u << shift;
            __syncthreads();
        }
    }
    // keys are unique (positions are), so "key >= the need-th largest" picks exactly `need`
    const uint64_t kth = prefix_s;
    const bool all = need >= ncand;
    if (need > 0) {
        const uint32_t n_iter = (ncand + kFinalThreads - 1) / kFinalThreads;
        for (uint32_t it = 0; it < n_iter; ++it) {
            const uint32_t i = it * kFinalThreads + t;
            bool take = false;
            int32_t pos = 0;
            if (i < ncand) {
                const uint64_t v = c[i];
                take = all || v >= kth;
                pos = (int32_t)(~(uint32_t)(v & 0xFFFFFFFFull));
            }
            wave_append<int32_t>(take, pos, &cursor, out, want);
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
    const unsigned nx = (unsigned)((capacity + kSelRowsPerBlock - 1) / kSelRowsPerBlock);
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
