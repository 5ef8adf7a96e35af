// append.hip -- quantise-append of a decode step's new entries.
//
// One workgroup per (new entry i, sequence b).  Each writes the quantised main
// row and indexer key at row slots[b, i] and, for i == 0, the bf16 window
// entry at ring slot win_pos[b] mod W.  The entry is quantised after RoPE with
// block scales only ([P1] "DeepSeek's Attention and KV Cache - From MLA to
// CSA2", "DeepSeek-V4.1", "Four bits for the main KV, eight for the window";
// 656 / 132-byte V3.2 rows: "DeepSeek-V3.2", "What it costs and what it
// saves").  Quantisation is bit-exact with the row-format definitions in
// mla.h: the block maximum, the fp32 divisions and the round-to-nearest-even
// encoders are the only arithmetic.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kThreads = 256;

// Quantise one row of `dim + rope` fp32 values into `dst` (row_bytes bytes).
// `amax_bits` is LDS scratch of at least dim/16 uints.
__device__ void quant_row(int fmt, int dim, int rope, const float* __restrict__ src,
                          uint8_t* __restrict__ dst, uint32_t* amax_bits) {
    const int t = threadIdx.x;
    if (fmt == MLA_FMT_F32) {
        for (int c = t; c < dim + rope; c += kThreads) reinterpret_cast<float*>(dst)[c] = src[c];
        return;
    }
    if (fmt == MLA_FMT_BF16) {
        for (int c = t; c < dim + rope; c += kThreads)
            reinterpret_cast<uint16_t*>(dst)[c] = (uint16_t)bf16_rne(src[c]);
        return;
    }
    const int blk = (fmt == MLA_FMT_E4M3_S128) ? 128 : 16;
    const int nblk = dim / blk;
    for (int j = t; j < nblk; j += kThreads) amax_bits[j] = 0u;
    __syncthreads();
    for (int c = t; c < dim; c += kThreads) atomicMax(&amax_bits[c / blk], f2u(fabsf(src[c])));
    __syncthreads();
    if (fmt == MLA_FMT_E4M3_S128) {
        float* scales = reinterpret_cast<float*>(dst + dim);     // dim is a multiple of 128
        for (int c = t; c < dim; c += kThreads) {
            const float a = u2f(amax_bits[c / 128]);
            const float s = a / 448.0f;
            dst[c] = (a == 0.0f) ? (uint8_t)0 : (uint8_t)e4m3_encode(src[c] / s);
        }
        for (int j = t; j < nblk; j += kThreads) scales[j] = u2f(amax_bits[j]) / 448.0f;
        uint16_t* ropep = reinterpret_cast<uint16_t*>(dst + dim + 4 * nblk);
        for (int r = t; r < rope; r += kThreads) ropep[r] = (uint16_t)bf16_rne(src[dim + r]);
    } else {  // MLA_FMT_E2M1_S16
        for (int p = t; p < dim / 2; p += kThreads) {
            const int c = 2 * p;
            const uint32_t sc = e4m3_encode(u2f(amax_bits[c / 16]) / 6.0f);
            const float sf = e4m3_to_f32(sc);
            uint32_t lo = 0u, hi = 0u;
            if (sf != 0.0f) {
                lo = e2m1_encode(src[c] / sf);
                hi = e2m1_encode(src[c + 1] / sf);
            }
            dst[p] = (uint8_t)(lo | (hi << 4));
        }
        for (int j = t; j < nblk; j += kThreads)
            dst[dim / 2 + j] = (uint8_t)e4m3_encode(u2f(amax_bits[j]) / 6.0f);
    }
}

__global__ __launch_bounds__(kThreads) void k_append(AppendArgs a) {
    __shared__ uint32_t amax_bits[64];          // dim/16 <= 64 (dim <= 1024)
    const int i = blockIdx.x, b = blockIdx.y;
    if ((a.main_cache || a.idx_cache) && i < a.n_new) {
        const int64_t slot = a.slots[(int64_t)b * a.n_new + i];
        if (slot >= 0 && slot < a.capacity) {
            if (a.main_cache) {
                const int D = a.main_dim + a.main_rope;
                quant_row(a.main_fmt, a.main_dim, a.main_rope, a.new_main + ((int64_t)b * a.n_new + i) * D,
                          a.main_cache + b * a.main_stride + slot * a.main_row_bytes, amax_bits);
                __syncthreads();
            }
            if (a.idx_cache) {
                quant_row(a.idx_fmt, a.idx_dim, 0, a.new_idx + ((int64_t)b * a.n_new + i) * a.idx_dim,
                          a.idx_cache + b * a.idx_stride + slot * a.idx_row_bytes, amax_bits);
            }
        }
    }
    if (a.win_ring && i == 0) {
        const int pos = a.win_pos[b];
        if (pos >= 0) {
            uint16_t* dst = a.win_ring + ((int64_t)b * a.W + pos % a.W) * a.Dw;
            const float* src = a.new_win + (int64_t)b * a.Dw;
            for (int c = threadIdx.x; c < a.Dw; c += kThreads) dst[c] = (uint16_t)bf16_rne(src[c]);
        }
    }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
    int n_blocks_x = (a.main_cache || a.idx_cache) ? a.n_new : 0;
    if (a.win_ring && n_blocks_x < 1) n_blocks_x = 1;
    if (a.B == 0 || n_blocks_x == 0) return hipSuccess;
    const ProfSlot p = prof_slot(PROF_APPEND);
    return launch_kernel(k_append, dim3(n_blocks_x, a.B), dim3(kThreads), 0, stream, p.start, p.stop, a);
}

}  // namespace mla
