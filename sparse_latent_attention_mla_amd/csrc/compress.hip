// compress.hip -- the CSA2 compressor at append, fused with the quantise-append.
//
// V4.1's compressor pools each window of m tokens into one entry, with windows
// that do not overlap and no position bias ([P1] "DeepSeek-V4.1", "CSA2: the
// simplified compressor"): a softmax of the gate over the window's tokens, per
// channel, weights the tokens' kv vectors; the sum is normalised (RMS, with a
// weight) ([P2] Part 2, the compressor's training-path code), the trailing
// RoPE channels are rotated at the window's position, and the entry is
// quantised into its main-cache row like any appended entry. The kv and gate
// projections, and the indexer key's projection from the entry, are the
// model's matmuls and stay with the caller.
#include "append.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kCompThreads = 256;

// One workgroup per sequence: thread t pools channels t, t + 256, ... over the
// m tokens (an online softmax). The loads of two tokens for all of a thread's
// channels, and the normalisation weights, are issued before any of them is
// used, so the window costs one memory round trip per two tokens; the mean
// square is a workgroup sum, the entry is normalised and rotated in LDS,
// written out in fp32 if asked, and quantised from LDS.
constexpr int kCompPer = kStageMain / kCompThreads;      // channels per thread, at most

__global__ __launch_bounds__(kCompThreads) void k_compress(CompressArgs a) {
    __shared__ float ent[kStageMain];
    __shared__ float red[kCompThreads / 64];
    __shared__ uint32_t amax_bits[64];
    const int b = blockIdx.x, t = threadIdx.x, D = a.D;
    const float* K = a.kv + (int64_t)b * a.m * D;
    const float* G = a.gate + (int64_t)b * a.m * D;
    const int64_t slot = a.slots ? a.slots[b] : -1;        // issued now, used at the end
    const int r = a.rope_dim, h = r / 2;
    float rcs[2] = {1.0f, 0.0f};                           // (cos, sin) of this thread's RoPE pair, if any
    if (t < h) {
        rcs[0] = a.rope_cs[((int64_t)b * h + t) * 2];
        rcs[1] = a.rope_cs[((int64_t)b * h + t) * 2 + 1];
    }
    float gw[kCompPer], mx[kCompPer], den[kCompPer], num[kCompPer];
#pragma unroll
    for (int j = 0; j < kCompPer; ++j) {
        const int c = t + kCompThreads * j;
        gw[j] = (c < D && a.g) ? a.g[c] : 1.0f;
        mx[j] = -__builtin_inff();
        den[j] = num[j] = 0.0f;
    }
    for (int i0 = 0; i0 < a.m; i0 += 2) {
        float gv[2][kCompPer], xv[2][kCompPer];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < kCompPer; ++j) {
                const int c = t + kCompThreads * j;
                const bool in = c < D && i0 + u < a.m;
                gv[u][j] = in ? G[(int64_t)(i0 + u) * D + c] : 0.0f;
                xv[u][j] = in ? K[(int64_t)(i0 + u) * D + c] : 0.0f;
            }
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < kCompPer; ++j) {
                if (t + kCompThreads * j >= D || i0 + u >= a.m) continue;
                if (gv[u][j] > mx[j]) {                      // new maximum: rescale what was summed
                    const float sc = expf(mx[j] - gv[u][j]);
                    den[j] = den[j] * sc + 1.0f;
                    num[j] = num[j] * sc + xv[u][j];
                    mx[j] = gv[u][j];
                } else {                                     // a gate of -inf weighs 0 (also while mx is -inf)
                    const float e = gv[u][j] == -__builtin_inff() ? 0.0f : expf(gv[u][j] - mx[j]);
                    den[j] += e;
                    num[j] += e * xv[u][j];
                }
            }
    }
    float ss = 0.0f;
#pragma unroll
    for (int j = 0; j < kCompPer; ++j) {
        const int c = t + kCompThreads * j;
        if (c < D) {
            const float p = num[j] / den[j];
            ent[c] = p;
            ss += p * p;
        }
    }
    ss = wave_sum(ss);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)D + a.eps);
#pragma unroll
    for (int j = 0; j < kCompPer; ++j) {
        const int c = t + kCompThreads * j;
        if (c < D) ent[c] = ent[c] * inv * gw[j];
    }
    __syncthreads();
    if (t < h) {                                           // one thread per RoPE pair (r <= 512: h <= 256)
        const float x1 = ent[D - r + t], x2 = ent[D - h + t];
        ent[D - r + t] = x1 * rcs[0] - x2 * rcs[1];
        ent[D - h + t] = x2 * rcs[0] + x1 * rcs[1];
    }
    __syncthreads();
    if (a.out)
        for (int c = t; c < D; c += kCompThreads) a.out[(int64_t)b * D + c] = ent[c];
    if (a.cache && slot >= 0 && slot < a.capacity)
        quant_row<kCompThreads>(a.fmt, a.dim, a.rope, ent, a.cache + b * a.stride + slot * a.row_bytes, amax_bits);
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return launch_kernel(k_compress, dim3(a.B), dim3(kCompThreads), 0, stream, nullptr, nullptr, a);
}

}  // namespace mla
