// indexer.hip -- lightning-indexer scan.
//
//   I[b, s] = sum_j w[b, j] * ReLU(sigma * q_idx[b, j, :] . k_idx[b, s, :])
// over one shared indexer key per cached row ([P1] "DeepSeek's Attention and
// KV Cache - From MLA to CSA2", "DeepSeek-V3.2", "The lightning indexer",
// eq. 1; [P2] "From MLA to DSA to HCA/CSA", Part 1, "The indexer"), with the
// causal mask (rows >= n_visible[b] are -inf, [P2] Part 2 "HCA").
//
// The scan is the HBM-bound streaming part of the step: every indexer row is
// read exactly once, coalesced, and dequantised in registers.  The
// (H_I x d_I) x (d_I x rows) contraction runs on bf16 MFMA (fp32 accumulate):
// E4M3 codes and E2M1 x E4M3-scale products are exact in bf16, so the keys
// enter the MFMA unrounded; the fp32 per-row scale of the E4M3 format is
// applied to the accumulator.  ReLU, the head weights and the head sum run on
// the accumulator in registers, and the top-k histogram of the score keys is
// built in LDS, so the only outputs are the fp32 scores and the histogram.
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kScanThreads = 256;         // 4 waves
constexpr int kTilesPerWave = 8;          // 16-row tiles per wave
constexpr int kRowsPerBlock = 4 * kTilesPerWave * 16;

// ------------------------------------------------------------------------
// Load the 32 channels g*32 .. g*32+31 of one indexer row as four bf16 MFMA
// B-operand chunks: kb[t] holds channels g*32 + t*8 .. +7.  Returns the
// post-contraction multiplier of the row (its fp32 scale for E4M3, else 1).
template <int FMT>
__device__ __forceinline__ float load_key_operand(const uint8_t* __restrict__ row, int g, u32x4 kb[4]) {
    if constexpr (FMT == MLA_FMT_BF16) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + g * 64);
#pragma unroll
        for (int t = 0; t < 4; ++t) kb[t] = __builtin_nontemporal_load(p + t);
        return 1.0f;
    } else if constexpr (FMT == MLA_FMT_E4M3_S128) {
        // 132-byte rows: 4-byte aligned only
        const uint32_t* p = reinterpret_cast<const uint32_t*>(row + g * 32);
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = __builtin_nontemporal_load(p + i);
        const float scale = __builtin_nontemporal_load(reinterpret_cast<const float*>(row + 128));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u32x2 lo = e4m3x4_to_bf16(w[2 * t]);
            u32x2 hi = e4m3x4_to_bf16(w[2 * t + 1]);
            kb[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
        return scale;
    } else {  // MLA_FMT_E2M1_S16, 72-byte rows: 8-byte aligned
        const u32x2* p = reinterpret_cast<const u32x2*>(row + g * 16);
        const u32x2 n01 = __builtin_nontemporal_load(p);
        const u32x2 n23 = __builtin_nontemporal_load(p + 1);
        const uint32_t sw = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(row + 64 + 2 * g));
        const float s0 = e4m3_to_f32(sw & 0xFFu), s1 = e4m3_to_f32(sw >> 8);
        const uint32_t nib[4] = {n01.x, n01.y, n23.x, n23.y};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float s = (t < 2) ? s0 : s1;
            const uint32_t w = nib[t];
            f32x2 v0 = e2m1x2_to_f32<0>(w), v1 = e2m1x2_to_f32<1>(w);
            f32x2 v2 = e2m1x2_to_f32<2>(w), v3 = e2m1x2_to_f32<3>(w);
            kb[t] = u32x4{pack_bf16_trunc(v0.x * s, v0.y * s), pack_bf16_trunc(v1.x * s, v1.y * s),
                          pack_bf16_trunc(v2.x * s, v2.y * s), pack_bf16_trunc(v3.x * s, v3.y * s)};
        }
        return 1.0f;
    }
}

// MFMA scan for d_I = 128 and H_I = 16 * MT.  Block: 4 waves, kRowsPerBlock rows
// of one sequence; a wave takes 16-row tiles.  Lane (col = l % 16, g = l / 16)
// owns row col of the tile and channels g*32 .. g*32+31 (k-slot (g, e) of
// k-step t is channel g*32 + t*8 + e, for A and B alike).
template <int FMT, int MT>
__global__ __launch_bounds__(kScanThreads) void k_scan_mfma(ScanArgs a) {
    __shared__ uint32_t hist[kHistBins];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int64_t nvis = clamp_visible(a.n_visible[b], a.capacity);
    const int64_t row0 = (int64_t)blockIdx.x * kRowsPerBlock;

    for (int i = threadIdx.x; i < kHistBins; i += kScanThreads) hist[i] = 0u;

    // A operand: q_idx of heads 16m + col, channels g*32 + t*8 .. +7
    u32x4 qa[MT][4];
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q_idx) + (int64_t)b * a.H_I * 128;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            qa[m][t] = *reinterpret_cast<const u32x4*>(qb + (16 * m + col) * 128 + g * 32 + t * 8);
    // head weights of the accumulator rows 4g + r of each head tile
    float wv[MT][4];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) wv[m][r] = a.w[(int64_t)b * a.H_I + 16 * m + 4 * g + r];
    __syncthreads();

    const uint8_t* base = a.cache + b * a.stride;
    float* scores = a.scores + b * a.capacity;
    for (int it = 0; it < kTilesPerWave; ++it) {
        const int64_t tile0 = row0 + (int64_t)(it * 4 + wave) * 16;
        if (tile0 >= a.capacity) break;
        const int64_t s = tile0 + col;
        const bool valid = s < nvis;
        if (tile0 >= nvis) {               // whole tile masked
            if (g == 0 && s < a.capacity) scores[s] = -__builtin_inff();
            continue;
        }
        u32x4 kb[4];
        float mult = 0.0f;
        if (valid) {
            mult = load_key_operand<FMT>(base + s * a.row_bytes, g, kb);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) kb[t] = u32x4{0u, 0u, 0u, 0u};
        }
        f32x4 acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = mfma_bf16(qa[m][t], kb[t], acc[m]);
        const float c = a.sigma * mult;
        float part = 0.0f;
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) part += wv[m][r] * fmaxf(acc[m][r] * c, 0.0f);
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        if (g == 0 && s < a.capacity) {
            scores[s] = valid ? part : -__builtin_inff();
            if (valid) atomicAdd(&hist[score_key(part) >> (32 - kHistBits)], 1u);
        }
    }
    __syncthreads();
    uint32_t* gh = a.hist + (int64_t)b * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kScanThreads) {
        const uint32_t v = hist[i];
        if (v) atomicAdd(&gh[i], v);
    }
}

// ------------------------------------------------------------------------
// Generic scan (any row format, any d_I, H_I * d_I <= 8192): one row per
// thread, fp32 FMA on the vector ALUs.  Used for shapes outside the MFMA
// specialisations (e.g. the tiny fp32 configuration).
__device__ __forceinline__ float e2m1_value(uint32_t n) {
    const uint32_t e = (n >> 1) & 3u, m = n & 1u;
    const float mag = e ? __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)e - 1) : 0.5f * (float)m;
    return (n & 8u) ? -mag : mag;
}

__device__ __forceinline__ float key_elem(int fmt, int dim, const uint8_t* row, int c) {
    switch (fmt) {
    case MLA_FMT_F32: return reinterpret_cast<const float*>(row)[c];
    case MLA_FMT_BF16: return u2f((uint32_t)reinterpret_cast<const uint16_t*>(row)[c] << 16);
    case MLA_FMT_E4M3_S128:
        return e4m3_to_f32(row[c]) * reinterpret_cast<const float*>(row + dim)[c / 128];
    default: {
        const uint32_t byte = row[c / 2];
        return e2m1_value((c & 1) ? (byte >> 4) : (byte & 15u)) * e4m3_to_f32(row[dim / 2 + c / 16]);
    }
    }
}

__global__ __launch_bounds__(kScanThreads) void k_scan_generic(ScanArgs a) {
    __shared__ float qs[8192];
    __shared__ uint32_t hist[kHistBins];
    const int b = blockIdx.y;
    const int n = a.H_I * a.dim;
    for (int i = threadIdx.x; i < n; i += kScanThreads) {
        qs[i] = (a.fmt == MLA_FMT_F32)
                    ? reinterpret_cast<const float*>(a.q_idx)[(int64_t)b * n + i]
                    : u2f((uint32_t)reinterpret_cast<const uint16_t*>(a.q_idx)[(int64_t)b * n + i] << 16);
    }
    for (int i = threadIdx.x; i < kHistBins; i += kScanThreads) hist[i] = 0u;
    __syncthreads();
    const int64_t s = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;
    const int64_t nvis = clamp_visible(a.n_visible[b], a.capacity);
    if (s < a.capacity) {
        float score = -__builtin_inff();
        if (s < nvis) {
            const uint8_t* row = a.cache + b * a.stride + s * a.row_bytes;
            score = 0.0f;
            for (int j = 0; j < a.H_I; ++j) {
                float d = 0.0f;
                for (int c = 0; c < a.dim; ++c) d += qs[j * a.dim + c] * key_elem(a.fmt, a.dim, row, c);
                score += a.w[(int64_t)b * a.H_I + j] * fmaxf(a.sigma * d, 0.0f);
            }
            atomicAdd(&hist[score_key(score) >> (32 - kHistBits)], 1u);
        }
        a.scores[b * a.capacity + s] = score;
    }
    __syncthreads();
    uint32_t* gh = a.hist + (int64_t)b * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kScanThreads) {
        const uint32_t v = hist[i];
        if (v) atomicAdd(&gh[i], v);
    }
}

}  // namespace

bool scan_supported(int fmt, int dim, int H_I) {
    if (H_I <= 0) return false;
    if ((fmt == MLA_FMT_BF16 || fmt == MLA_FMT_E4M3_S128 || fmt == MLA_FMT_E2M1_S16) && dim == 128 &&
        H_I % 16 == 0 && H_I <= 64)
        return true;
    return H_I * dim <= 8192;
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
    if (a.B == 0 || a.capacity == 0) return hipSuccess;
    const bool mfma = (a.fmt == MLA_FMT_BF16 || a.fmt == MLA_FMT_E4M3_S128 || a.fmt == MLA_FMT_E2M1_S16) &&
                      a.dim == 128 && a.H_I % 16 == 0 && a.H_I <= 64;
    if (mfma) {
        const dim3 grid((unsigned)((a.capacity + kRowsPerBlock - 1) / kRowsPerBlock), a.B);
#define MLA_SCAN_CASE(F, M)                                                              \
    if (a.fmt == F && a.H_I == 16 * M) {                                                 \
        hipLaunchKernelGGL((k_scan_mfma<F, M>), grid, dim3(kScanThreads), 0, stream, a); \
        return hipGetLastError();                                                        \
    }
        MLA_SCAN_CASE(MLA_FMT_BF16, 1) MLA_SCAN_CASE(MLA_FMT_BF16, 2)
        MLA_SCAN_CASE(MLA_FMT_BF16, 3) MLA_SCAN_CASE(MLA_FMT_BF16, 4)
        MLA_SCAN_CASE(MLA_FMT_E4M3_S128, 1) MLA_SCAN_CASE(MLA_FMT_E4M3_S128, 2)
        MLA_SCAN_CASE(MLA_FMT_E4M3_S128, 3) MLA_SCAN_CASE(MLA_FMT_E4M3_S128, 4)
        MLA_SCAN_CASE(MLA_FMT_E2M1_S16, 1) MLA_SCAN_CASE(MLA_FMT_E2M1_S16, 2)
        MLA_SCAN_CASE(MLA_FMT_E2M1_S16, 3) MLA_SCAN_CASE(MLA_FMT_E2M1_S16, 4)
#undef MLA_SCAN_CASE
        return hipErrorInvalidValue;
    }
    const dim3 grid((unsigned)((a.capacity + kScanThreads - 1) / kScanThreads), a.B);
    hipLaunchKernelGGL(k_scan_generic, grid, dim3(kScanThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace mla
