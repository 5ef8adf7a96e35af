// pool.hip -- block maxima for the candidate pool of the hierarchical sparse indexer.
//
// A Full layer that publishes a candidate pool ([P4] "The Hierarchical
// Sparse Indexer: bounded sweeps"; [P1] "DeepSeek-V4.1", "The hierarchical
// indexer") groups its visible positions into blocks of `block` consecutive
// positions, scores each block by the largest score inside it, and keeps the
// best blocks; the deeper (Reindex) layers then score only those blocks'
// positions.  This kernel computes the block scores and the 12-bit key
// histogram the radix selection starts from; the selection itself is the
// top-k's (launch_select over the block scores, reporting every selected
// block's positions).
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kPoolThreads = 256;
constexpr int kPoolIters = 16;            // 64-position strips per wave
constexpr int kPoolRows = kPoolThreads * kPoolIters;   // positions per workgroup

// Lanes read consecutive scores (one coalesced load per 64 positions), and the
// `block` lanes of a block (block a power of two <= 64) meet in a butterfly
// maximum; invisible positions enter as -inf.  The block score is canonicalised
// (+0 for a zero maximum) so that its key orders like the float comparison.
__global__ __launch_bounds__(kPoolThreads) void k_block_max(const float* __restrict__ scores, int64_t capacity,
                                                            const int32_t* __restrict__ n_visible, int block,
                                                            int lg_block, float* __restrict__ bmax,
                                                            int32_t* __restrict__ nvb, uint32_t* __restrict__ hist_all) {
    __shared__ uint32_t hist[kHistBins];
    const int b = blockIdx.y;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int64_t nvis = clamp_visible(n_visible[b], capacity);
    const int64_t nb_cap = (capacity + block - 1) >> lg_block;
    const int64_t n_vb = (nvis + block - 1) >> lg_block;
    const int64_t r0 = (int64_t)blockIdx.x * kPoolRows + (int64_t)wave * 64 * kPoolIters;
    const float* sc = scores + b * capacity;
    float v[kPoolIters];
#pragma unroll
    for (int i = 0; i < kPoolIters; ++i) {
        const int64_t s = r0 + 64 * i + lane;
        v[i] = (s < nvis) ? sc[s] : -__builtin_inff();
    }
    for (int i = t; i < kHistBins; i += kPoolThreads) hist[i] = 0u;
    if (blockIdx.x == 0 && t == 0) nvb[b] = (int32_t)n_vb;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kPoolIters; ++i) {
        float m = v[i];
        for (int w = 1; w < block; w <<= 1) {
            const float o = __shfl_xor(m, w, 64);
            m = (o > m) ? o : m;
        }
        const int64_t s = r0 + 64 * i + lane;
        const int64_t blk = s >> lg_block;
        if ((lane & (block - 1)) == 0 && blk < nb_cap) {
            m = m + 0.0f;                                   // -0 -> +0
            bmax[b * nb_cap + blk] = m;
            if (blk < n_vb) atomicAdd(&hist[score_key(m) >> (32 - kHistBits)], 1u);
        }
    }
    __syncthreads();
    flush_hist_copy([&](int i) { return hist[i]; }, hist_all + (int64_t)b * kHistWordsHost, hist_copy_of_block(),
                    kPoolThreads);
}

}  // namespace

hipError_t launch_block_max(const float* scores, int64_t capacity, const int32_t* n_visible, int B, int block,
                            float* bmax, int32_t* nvb, uint32_t* hist, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    int lg = 0;
    while ((1 << lg) < block) ++lg;
    if ((1 << lg) != block || block > 64) return hipErrorInvalidValue;
    const unsigned gx = (unsigned)std::max<int64_t>(1, (capacity + kPoolRows - 1) / kPoolRows);
    return launch_kernel(k_block_max, dim3(gx, B), dim3(kPoolThreads), 0, stream, nullptr, nullptr, scores,
                         capacity, n_visible, block, lg, bmax, nvb, hist);
}

}  // namespace mla
