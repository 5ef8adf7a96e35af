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

constexpr int kStageMain = 2048;           // rows up to these sizes are staged through LDS
constexpr int kStageIdx = 1024;

// Every global load of the block (slot, new rows, window entry) is issued at
// entry, before any of them is used, so the block pays one memory round trip;
// the rows then wait in LDS for the quantisers.
__global__ __launch_bounds__(kThreads) void k_append(AppendArgs a) {
    __shared__ uint32_t amax_bits[64];          // dim/16 <= 64 (dim <= 1024), dim/128 <= 64
    __shared__ float s_main[kStageMain];
    __shared__ float s_idx[kStageIdx];
    const int i = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const bool rows = (a.main_cache || a.idx_cache) && i < a.n_new;
    const int D = a.main_dim + a.main_rope;
    const int64_t e = (int64_t)b * a.n_new + i;
    const float* gmain = (rows && a.main_cache) ? a.new_main + e * D : nullptr;
    const float* gidx = (rows && a.idx_cache) ? a.new_idx + e * a.idx_dim : nullptr;
    const bool stage = D <= kStageMain && a.idx_dim <= kStageIdx;
    const int64_t slot = rows ? a.slots[e] : -1;
    float vm[kStageMain / kThreads], vi[kStageIdx / kThreads];
    if (stage) {
#pragma unroll
        for (int j = 0; j < kStageMain / kThreads; ++j) {
            const int c = t + kThreads * j;
            vm[j] = (gmain && c < D) ? gmain[c] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kStageIdx / kThreads; ++j) {
            const int c = t + kThreads * j;
            vi[j] = (gidx && c < a.idx_dim) ? gidx[c] : 0.0f;
        }
    }
    const bool win = a.win_ring && i == 0;
    const int pos = win ? a.win_pos[b] : -1;
    const float* wsrc = a.new_win + (int64_t)b * a.Dw;
    float vw[kStageMain / kThreads];
    const bool wstage = win && a.Dw <= kStageMain;
    if (wstage) {
#pragma unroll
        for (int j = 0; j < kStageMain / kThreads; ++j) {
            const int c = t + kThreads * j;
            vw[j] = (c < a.Dw) ? wsrc[c] : 0.0f;
        }
    }
    if (stage) {
#pragma unroll
        for (int j = 0; j < kStageMain / kThreads; ++j) s_main[t + kThreads * j] = vm[j];
#pragma unroll
        for (int j = 0; j < kStageIdx / kThreads; ++j) s_idx[t + kThreads * j] = vi[j];
        __syncthreads();
    }
    if (rows && slot >= 0 && slot < a.capacity) {
        if (gmain) {
            quant_row(a.main_fmt, a.main_dim, a.main_rope, stage ? s_main : gmain,
                      a.main_cache + b * a.main_stride + slot * a.main_row_bytes, amax_bits);
            __syncthreads();
        }
        if (gidx)
            quant_row(a.idx_fmt, a.idx_dim, 0, stage ? s_idx : gidx,
                      a.idx_cache + b * a.idx_stride + slot * a.idx_row_bytes, amax_bits);
    }
    if (win && pos >= 0) {
        uint16_t* dst = a.win_ring + ((int64_t)b * a.W + pos % a.W) * a.Dw;
        if (wstage) {
#pragma unroll
            for (int j = 0; j < kStageMain / kThreads; ++j) {
                const int c = t + kThreads * j;
                if (c < a.Dw) dst[c] = (uint16_t)bf16_rne(vw[j]);
            }
        } else {
            for (int c = t; c < a.Dw; c += kThreads) dst[c] = (uint16_t)bf16_rne(wsrc[c]);
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
