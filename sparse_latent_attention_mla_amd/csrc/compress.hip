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
// m tokens (an online softmax: one pass over the gates and kv, coalesced per
// token), the mean square is a workgroup sum, the entry is normalised and
// rotated in LDS, written out in fp32 if asked, and quantised from LDS.
__global__ __launch_bounds__(kCompThreads) void k_compress(CompressArgs a) {
    __shared__ float ent[kStageMain];
    __shared__ float red[kCompThreads / 64];
    __shared__ uint32_t amax_bits[64];
    const int b = blockIdx.x, t = threadIdx.x, D = a.D;
    const float* K = a.kv + (int64_t)b * a.m * D;
    const float* G = a.gate + (int64_t)b * a.m * D;
    float ss = 0.0f;
    for (int c = t; c < D; c += kCompThreads) {
        float mx = -__builtin_inff(), den = 0.0f, num = 0.0f;
        for (int i = 0; i < a.m; ++i) {
            const float gv = G[(int64_t)i * D + c], x = K[(int64_t)i * D + c];
            if (gv > mx) {                                   // new maximum: rescale what was summed
                const float s = expf(mx - gv);
                den = den * s + 1.0f;
                num = num * s + x;
                mx = gv;
            } else {
                const float e = expf(gv - mx);
                den += e;
                num += e * x;
            }
        }
        const float p = num / den;
        ent[c] = p;
        ss += p * p;
    }
    ss = wave_sum(ss);
    if ((t & 63) == 0) red[t >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf(((red[0] + red[1]) + (red[2] + red[3])) / (float)D + a.eps);
    for (int c = t; c < D; c += kCompThreads) ent[c] = ent[c] * inv * (a.g ? a.g[c] : 1.0f);
    __syncthreads();
    const int r = a.rope_dim, h = r / 2;
    for (int i = t; i < h; i += kCompThreads) {             // one thread per RoPE pair
        const float cs = a.rope_cs[((int64_t)b * h + i) * 2], sn = a.rope_cs[((int64_t)b * h + i) * 2 + 1];
        const float x1 = ent[D - r + i], x2 = ent[D - h + i];
        ent[D - r + i] = x1 * cs - x2 * sn;
        ent[D - h + i] = x2 * cs + x1 * sn;
    }
    __syncthreads();
    if (a.out)
        for (int c = t; c < D; c += kCompThreads) a.out[(int64_t)b * D + c] = ent[c];
    const int64_t slot = a.slots ? a.slots[b] : -1;
    if (a.cache && slot >= 0 && slot < a.capacity)
        quant_row<kCompThreads>(a.fmt, a.dim, a.rope, ent, a.cache + b * a.stride + slot * a.row_bytes, amax_bits);
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return launch_kernel(k_compress, dim3(a.B), dim3(kCompThreads), 0, stream, nullptr, nullptr, a);
}

}  // namespace mla
