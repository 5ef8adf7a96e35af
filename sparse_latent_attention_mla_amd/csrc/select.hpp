// select.hpp -- pieces of the radix selection shared by the top-k kernels and by the
// decode that finishes a selection from k_select's lists: wave prefix sums, the digit
// search over a histogram, the threshold bin of a sequence's score histogram, and the
// zeroing of that histogram for the next call.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kMaxDigitBins = 1024;

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Inclusive prefix sum over the lanes of a wave, on DPP: shifts by 1, 2, 4, 8 within
// each row of 16 lanes, then row 0's (row 1's) last lane added to rows 1, 3 (2, 3).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

// Zero sequence b's histogram (all copies) once its threshold has been read, so
// that the next call's scan finds it cleared. Called by every thread of a block.
__device__ __forceinline__ void zero_hist(uint32_t* hb) {
    u32x4* p = reinterpret_cast<u32x4*>(hb);
    for (int i = threadIdx.x; i < (int)(kHistWordsHost / 4); i += blockDim.x) p[i] = u32x4{0u, 0u, 0u, 0u};
}

// The sum over the copies of coarse bin 63 - lane (the first wave of a block;
// loaded early, used by zero_hist_rest).
__device__ __forceinline__ uint32_t coarse_sum_of_lane(const uint32_t* hb) {
    const int lane = threadIdx.x & 63;
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kHistCopies; ++j) sum += hist_coarse(const_cast<uint32_t*>(hb), j)[kCoarseBins - 1 - lane];
    return sum;
}

// What k_select leaves of the zeroing: the coarse level and, when there is a
// threshold, the fine bins of its coarse bin (found again from the coarse level,
// as the threshold search does; `sum`: coarse_sum_of_lane, for the first wave).
// Called by every thread of a block of >= 128.
__device__ __forceinline__ void zero_hist_rest(uint32_t* hb, uint32_t need, uint32_t sum) {
    __shared__ int cb_s;
    const int t = threadIdx.x, lane = t & 63;
    if (t < 64) {
        const uint32_t incl = wave_incl_scan(sum), excl = incl - sum;
        const uint64_t hit = __ballot(excl < need && incl >= need);
        if (t == 0) cb_s = hit ? kCoarseBins - 1 - __builtin_ctzll(hit) : -1;
    }
    lds_barrier();
    const int cb = cb_s;
    if (cb >= 0 && t < kHistCopies * kFinePerCoarse / 4)       // 8 copies x 64 bins, 4 per thread
        reinterpret_cast<u32x4*>(hist_fine(hb, t / (kFinePerCoarse / 4)) + cb * kFinePerCoarse)[t % (kFinePerCoarse / 4)] =
            u32x4{0u, 0u, 0u, 0u};
    if (t < kHistCopies * kCoarseBins / 4) reinterpret_cast<u32x4*>(hb)[t] = u32x4{0u, 0u, 0u, 0u};
}

// Digit search by one wave over counts h[0 .. nbins) (nbins 256 or 1024; global or LDS):
// lane l holds the bins nbins-1-l*per .. nbins-(l+1)*per in registers (largest first).
// Finds d with sum_{e>d} h[e] < need <= sum_{e>=d} h[e]; found = false when the total is
// below need. Results are uniform across the wave.
struct DigitResult {
    int digit;
    uint32_t above, count;
    bool found;
};
template <typename P>
__device__ __forceinline__ DigitResult wave_find_digit(P h, int nbins, uint32_t need) {
    const int lane = threadIdx.x & 63;
    const int per = nbins >> 6;                           // 4 or 16
    const int lo = nbins - (lane + 1) * per;              // the lane's bins lo .. lo + per - 1
    uint32_t hv[16];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
        u32x4 q = u32x4{0u, 0u, 0u, 0u};
        if (i < per) q = *reinterpret_cast<const u32x4*>(&h[lo + i]);
        hv[i] = q.x;
        hv[i + 1] = q.y;
        hv[i + 2] = q.z;
        hv[i + 3] = q.w;
        sum += q.x + q.y + q.z + q.w;
    }
    const uint32_t incl = wave_incl_scan(sum), excl = incl - sum;
    const uint64_t hit = __ballot(excl < need && incl >= need);
    DigitResult r{0, 0u, 0u, hit != 0};
    if (!r.found) return r;
    const int src = __builtin_ctzll(hit);
    // every lane walks its own bins down from the top; the hit lane's result is read out
    int d = 0;
    uint32_t above = 0, cnt = 0, run = excl;
    bool done = false;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
        if (i < per && !done) {
            const uint32_t c = hv[i];
            if (run + c >= need) {
                d = lo + i;
                above = run;
                cnt = c;
                done = true;
            } else {
                run += c;
            }
        }
    }
    r.digit = __builtin_amdgcn_readlane(d, src);
    r.above = (uint32_t)__builtin_amdgcn_readlane((int)above, src);
    r.count = (uint32_t)__builtin_amdgcn_readlane((int)cnt, src);
    return r;
}

// The threshold bin of sequence b's histogram (fine bin d with sum_{e>d} < need
// <= sum_{e>=d}; found = false when the total is below need), by one wave: lane l
// sums the copies of coarse bin 63 - l, a prefix sum finds the coarse bin, then
// the same over its 64 fine bins. Results are uniform across the wave.
__device__ __forceinline__ DigitResult hist_find(uint32_t* hb, uint32_t need) {
    const int lane = threadIdx.x & 63;
    uint32_t sum = 0;
#pragma unroll
    for (int j = 0; j < kHistCopies; ++j) sum += hist_coarse(hb, j)[kCoarseBins - 1 - lane];
    uint32_t incl = wave_incl_scan(sum), excl = incl - sum;
    uint64_t hit = __ballot(excl < need && incl >= need);
    DigitResult r{0, 0u, 0u, hit != 0};
    if (!r.found) return r;
    int src = __builtin_ctzll(hit);
    const int cb = kCoarseBins - 1 - src;
    const uint32_t above_c = (uint32_t)__builtin_amdgcn_readlane((int)excl, src);
    sum = 0;
#pragma unroll
    for (int j = 0; j < kHistCopies; ++j) sum += hist_fine(hb, j)[cb * kFinePerCoarse + kFinePerCoarse - 1 - lane];
    incl = wave_incl_scan(sum);
    excl = incl - sum;
    hit = __ballot(above_c + excl < need && above_c + incl >= need);
    src = __builtin_ctzll(hit);                            // found: the coarse bin holds the need-th key
    r.digit = cb * kFinePerCoarse + kFinePerCoarse - 1 - src;
    r.above = above_c + (uint32_t)__builtin_amdgcn_readlane((int)excl, src);
    r.count = (uint32_t)__builtin_amdgcn_readlane((int)sum, src);
    return r;
}

}  // namespace

}  // namespace mla
