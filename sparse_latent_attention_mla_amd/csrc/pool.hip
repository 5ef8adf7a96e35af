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
constexpr int kPoolPer = 2;               // blocks per thread
constexpr int kPoolBlocks = kPoolThreads * kPoolPer;   // blocks per workgroup

// Each thread scores whole blocks (consecutive threads, consecutive blocks):
// it loads the block's scores (16-byte vectors when the rows allow), takes their
// maximum over the visible positions (invisible ones enter as -inf) and adds the
// block score's key to the workgroup's LDS histogram. The block score is
// canonicalised (+0 for a zero maximum) so that its key orders like the float
// comparison.
template <bool VEC4>
__global__ __launch_bounds__(kPoolThreads) void k_block_max(const float* __restrict__ scores, int64_t capacity,
                                                            const int32_t* __restrict__ n_visible, int block,
                                                            int lg_block, float* __restrict__ bmax,
                                                            int32_t* __restrict__ nvb, uint32_t* __restrict__ hist_all) {
    __shared__ uint32_t hist[kHistBins];
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int64_t nvis = clamp_visible(n_visible[b], capacity);
    const int64_t nb_cap = (capacity + block - 1) >> lg_block;
    const int64_t n_vb = (nvis + block - 1) >> lg_block;
    const float* sc = scores + b * capacity;
    float m[kPoolPer];
#pragma unroll
    for (int u = 0; u < kPoolPer; ++u) {
        const int64_t blk = (int64_t)blockIdx.x * kPoolBlocks + u * kPoolThreads + t;
        const int64_t s0 = blk << lg_block;
        float x = -__builtin_inff();
        if (blk < n_vb) {
            if constexpr (VEC4) {
                for (int j = 0; j < block && s0 + j < nvis; j += 4) {   // (then all 4 lie below capacity)
                    const f32x4 q = *reinterpret_cast<const f32x4*>(sc + s0 + j);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (s0 + j + e < nvis && q[e] > x) x = q[e];
                }
            } else {
                for (int j = 0; j < block; ++j)
                    if (s0 + j < nvis && sc[s0 + j] > x) x = sc[s0 + j];
            }
        }
        m[u] = x + 0.0f;                                    // -0 -> +0
    }
    for (int i = t; i < kHistBins; i += kPoolThreads) hist[i] = 0u;
    if (blockIdx.x == 0 && t == 0) nvb[b] = (int32_t)n_vb;
    lds_barrier();
#pragma unroll
    for (int u = 0; u < kPoolPer; ++u) {
        const int64_t blk = (int64_t)blockIdx.x * kPoolBlocks + u * kPoolThreads + t;
        if (blk < nb_cap) bmax[b * nb_cap + blk] = m[u];
        if (blk < n_vb) atomicAdd(&hist[score_key(m[u]) >> (32 - kHistBits)], 1u);
    }
    lds_barrier();
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
    const int64_t nb = (capacity + block - 1) >> lg;
    const unsigned gx = (unsigned)std::max<int64_t>(1, (nb + kPoolBlocks - 1) / kPoolBlocks);
    // 16-byte loads when every block starts 16-byte aligned
    const bool vec4 = block % 4 == 0 && capacity % 4 == 0 && reinterpret_cast<uintptr_t>(scores) % 16 == 0;
    if (vec4)
        return launch_kernel(k_block_max<true>, dim3(gx, B), dim3(kPoolThreads), 0, stream, nullptr, nullptr,
                             scores, capacity, n_visible, block, lg, bmax, nvb, hist);
    return launch_kernel(k_block_max<false>, dim3(gx, B), dim3(kPoolThreads), 0, stream, nullptr, nullptr, scores,
                         capacity, n_visible, block, lg, bmax, nvb, hist);
}

}  // namespace mla
