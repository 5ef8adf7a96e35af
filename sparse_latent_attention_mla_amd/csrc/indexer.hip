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
#include <algorithm>
#include <cstdlib>

#include "append.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

// A row's score as the selection sees it: the fp32 score, or (the bf16-score top-k,
// [P1] "DeepSeek-V4", "The indexer in four bits") that score rounded to bf16, round to
// nearest even; -inf stays -inf.
__device__ __forceinline__ float sel_score(float s, int bf16) { return bf16 ? u2f(bf16_rne(s) << 16) : s; }


constexpr int kScanThreads = 256;         // 4 waves
constexpr int kTilesPerWave = 8;          // 16-row tiles per wave (direct-load path)
constexpr int kRowsPerBlock = 4 * kTilesPerWave * 16;
constexpr int kChunkRows = 64;            // rows a wave stages through LDS per step
constexpr int kStagedBlocks = 512;        // target workgroups of the staged scan (2 per CU)
constexpr int kDmaRows = 32;              // rows per chunk of the LDS-DMA scan
constexpr int kDmaMaxRowsPerBlock = 1024;
constexpr int kDmaRowsPerWave = 256;      // rows of a block per wave, at most (32x32 scan)
#ifndef MLA_SCAN_RPW4
#define MLA_SCAN_RPW4 512
#endif
constexpr int kDmaRowsPerWave4 = MLA_SCAN_RPW4;   // the same for the four-bit keys (68 and 72 B rows)
#ifndef MLA_SCAN_NBUF4
#define MLA_SCAN_NBUF4 2
#endif
constexpr int kDmaNbuf4 = MLA_SCAN_NBUF4;          // ring depth of the 32x32 scan for the four-bit keys
template <int FMT>
constexpr int dma32_chunk_rows() { return FMT == MLA_FMT_E4M3_S128 ? kDmaRows : 2 * kDmaRows; }
template <int FMT>
constexpr int dma32_rows_per_wave() { return FMT == MLA_FMT_E4M3_S128 ? kDmaRowsPerWave : kDmaRowsPerWave4; }
#ifndef MLA_SCAN_WAVES
#define MLA_SCAN_WAVES 4                  // waves per block of the 32x32 scan (4 or 8)
#endif
constexpr int kDma32Waves = MLA_SCAN_WAVES;
#ifndef MLA_SCAN_NBUF
#define MLA_SCAN_NBUF 2                   // chunk buffers per wave in the LDS-DMA scan
#endif
constexpr int kDmaNbuf = MLA_SCAN_NBUF;
constexpr int kDmaBlocksPerCu = (kDmaNbuf == 2) ? 3 : 2;   // what the LDS of one CU holds
#ifndef MLA_SCAN_STATIC_JOBS
#define MLA_SCAN_STATIC_JOBS 4
#endif
constexpr int kScanStaticJobs = MLA_SCAN_STATIC_JOBS;      // queue-fed scan: chunks per wave by index

typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Dequantise the 32 channels g*32 .. g*32+31 of a row (given as raw words) into
// four bf16 MFMA B-operand chunks kb[t] = channels g*32 + t*8 .. +7.
template <int FMT>
__device__ __forceinline__ void dequant_key(const uint32_t* w, uint32_t sw, u32x4 kb[4]) {
    if constexpr (FMT == MLA_FMT_E4M3_S128) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u32x2 lo = e4m3x4_to_bf16(w[2 * t]);
            u32x2 hi = e4m3x4_to_bf16(w[2 * t + 1]);
            kb[t] = u32x4{lo.x, lo.y, hi.x, hi.y};
        }
    } else {  // E2M1 x E4M3 scale (x E8M0 scale for MXFP4: one per 32 channels), exact in bf16
        const float s0 = FMT == MLA_FMT_MXFP4 ? e8m0_to_f32(sw & 0xFFu) : e4m3_to_f32(sw & 0xFFu);
        const float s1 = FMT == MLA_FMT_MXFP4 ? s0 : e4m3_to_f32((sw >> 8) & 0xFFu);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float s = (t < 2) ? s0 : s1;
            f32x2 v0 = e2m1x2_to_f32<0>(w[t]), v1 = e2m1x2_to_f32<1>(w[t]);
            f32x2 v2 = e2m1x2_to_f32<2>(w[t]), v3 = e2m1x2_to_f32<3>(w[t]);
            kb[t] = u32x4{pack_bf16_trunc(v0.x * s, v0.y * s), pack_bf16_trunc(v1.x * s, v1.y * s),
                          pack_bf16_trunc(v2.x * s, v2.y * s), pack_bf16_trunc(v3.x * s, v3.y * s)};
        }
    }
}

// The same 32 channels of an E2M1 x E4M3-scale row widened to fp16 for the
// f16 MFMA: every product of an E2M1 value (at most 2 significant bits, 0.5 .. 6)
// and an E4M3 scale (at most 4 bits, 2^-9 .. 448) lies in fp16's normal range
// with at most 5 significant bits, so the packed fp16 multiply is exact.
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
__device__ __forceinline__ void dequant_e2m1_f16(const uint32_t* w, uint32_t sw, u32x4 kb[4]) {
    const _Float16 s0 = (_Float16)e4m3_to_f32(sw & 0xFFu), s1 = (_Float16)e4m3_to_f32((sw >> 8) & 0xFFu);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const f16x2 s = (t < 2) ? f16x2{s0, s0} : f16x2{s1, s1};
        kb[t] = u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[t], 1.0f, 0) * s),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[t], 1.0f, 1) * s),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[t], 1.0f, 2) * s),
                      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[t], 1.0f, 3) * s)};
    }
}

// A query head held as bf16 pairs (u32x4 of 8 values) moved to fp16 after
// scaling by 2^k: exact for every value within 2^32 of the head's largest
// (k puts that largest in [2^14, 2^15)); smaller ones round to fp16's grid.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8_scaled(u32x4 q, float p) {
    u32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const f16x2 v = {(_Float16)(u2f(q[e] << 16) * p), (_Float16)(u2f(q[e] & 0xFFFF0000u) * p)};
        r[e] = __builtin_bit_cast(uint32_t, v);
    }
    return r;
}

// Bytes of a 128-channel indexer row of format FMT.
template <int FMT>
constexpr int idx_rb() {
    return FMT == MLA_FMT_E4M3_S128 ? 132 : (FMT == MLA_FMT_MXFP4 ? 68 : 72);
}

// The MXFP4 rounding of one query block of 32 channels, held as four vectors
// of 8 bf16 values, in place: the block's E8M0 code from its largest magnitude,
// E2M1 elements, values back in bf16 (exact: a rung times a power of two). With
// MXFP4 keys the query-key product is FP4 on both sides ([P1] "DeepSeek-V4",
// "The indexer in four bits"). Round-to-nearest-even on the E2M1 ladder is
// rint on its grid of the binade: steps of 1/2 below 2, of 1 below 4, of 2
// above (saturating at 6) -- the nearest rung, ties to the even code.
__device__ __forceinline__ void mx_round_query(u32x4* q) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = max(m, max((q[i][e] << 16) & 0x7FFFFFFFu, q[i][e] & 0x7FFF0000u));
    const uint32_t code = mx_code(m);
    const float X = e8m0_to_f32(code);
    const int sh = 127 - (int)code;
    auto round1 = [&](uint32_t bits) -> uint32_t {            // fp32 bits of a bf16 value -> rounded bf16
        const float a = __builtin_ldexpf(u2f(bits & 0x7FFFFFFFu), sh);     // |x| / X, exact, < 8
        const float step = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);
        const float inv = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
        const float r = fminf(__builtin_rintf(a * inv) * step, 6.0f);
        return ((f2u(r * X) >> 16) & 0x7FFFu) | ((bits >> 16) & 0x8000u);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) q[i][e] = round1(q[i][e] << 16) | (round1(q[i][e] & 0xFFFF0000u) << 16);
}

// The same rounding of one query block kept as MX codes for the FP4 MFMA: the
// 32 E2M1 codes (channel 2i in the low nibble of byte i; the rung r is code
// 2r below 2, r + 2 below 4, r / 2 + 4 above, the sign in bit 3) into `codes`,
// the block's E8M0 code returned.
__device__ __forceinline__ uint32_t mx_encode_query(const u32x4* q, u32x4& codes) {
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) m = max(m, max((q[i][e] << 16) & 0x7FFFFFFFu, q[i][e] & 0x7FFF0000u));
    const uint32_t code = mx_code(m);
    const int sh = 127 - (int)code;
    auto enc1 = [&](uint32_t bits) -> uint32_t {              // fp32 bits of a bf16 value -> E2M1 code
        const float a = __builtin_ldexpf(u2f(bits & 0x7FFFFFFFu), sh);
        const float step = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);
        const float inv = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
        const float r = fminf(__builtin_rintf(a * inv) * step, 6.0f);
        const uint32_t c = r < 2.0f ? (uint32_t)(2.0f * r) : (r < 4.0f ? (uint32_t)r + 2u : (uint32_t)(0.5f * r) + 4u);
        return c | ((bits >> 28) & 8u);
    };
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w |= (enc1(q[i][e] << 16) | (enc1(q[i][e] & 0xFFFF0000u) << 4)) << (8 * e);
        codes[i] = w;
    }
    return code;
}

// ReLU on the bit pattern: a set sign bit is a negative int32 (also for -0),
// so the signed integer max with 0 clears it; one instruction, no NaN canonicalisation.
__device__ __forceinline__ float relu(float x) {
    return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

template <int MT>
struct ScanCtx {
    u32x4 qa[MT][4];      // A operand: q_idx of heads 16m + col, channels g*32 + t*8 .. +7
    float wv[MT][4];      // w * sigma of accumulator rows 4g + r of head tile m
};

// Contract one 16-row tile: lane (col, g) holds the B operand of row col of
// the tile; returns that row's score (every g holds it); `mult` is the row's
// post-contraction factor.
template <int MT>
__device__ __forceinline__ float tile_epilogue(const ScanCtx<MT>& C, const f32x4 acc[MT], float mult);
template <int MT>
__device__ __forceinline__ float tile_dot(const ScanCtx<MT>& C, const u32x4 kb[4], float mult) {
    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = mfma_bf16(C.qa[m][t], kb[t], acc[m]);
    return tile_epilogue<MT>(C, acc, mult);
}

// The row's score from its tile accumulators (every g holds it).
template <int MT>
__device__ __forceinline__ float tile_epilogue(const ScanCtx<MT>& C, const f32x4 acc[MT], float mult) {
    // sum_j w_j ReLU(sigma * mult * d_j) = mult * sum_j (w_j sigma) ReLU(d_j)  (sigma, mult >= 0)
    float pm[MT];                                         // one partial sum per head tile: short chains
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        pm[m] = C.wv[m][0] * relu(acc[m][0]);
#pragma unroll
        for (int r = 1; r < 4; ++r) pm[m] += C.wv[m][r] * relu(acc[m][r]);
    }
    float part = pm[0];
#pragma unroll
    for (int m = 1; m < MT; ++m) part += pm[m];
    return xsum4(part) * mult;
}

// Contract one 16-row tile and emit its scores: row `s` (= tile0 + col).
template <int MT>
__device__ __forceinline__ void tile_scores(const ScanCtx<MT>& C, const u32x4 kb[4], float mult, int64_t s,
                                            bool valid, int g, float sigma, int64_t capacity, float* scores,
                                            uint32_t* hist, int round16) {
    const float part = sel_score(tile_dot<MT>(C, kb, mult), round16);
    if (g == 0 && s < capacity) {
        scores[s] = valid ? part : -__builtin_inff();
        if (valid) atomicAdd(&hist[score_key(part) >> (32 - kHistBits)], 1u);
    }
}

template <int MT>
__device__ __forceinline__ void load_ctx(ScanCtx<MT>& C, const ScanArgs& a, int b, int col, int g) {
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q_idx) + (int64_t)b * a.H_I * 128;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            C.qa[m][t] = *reinterpret_cast<const u32x4*>(qb + (16 * m + col) * 128 + g * 32 + t * 8);
    if (a.fmt == MLA_FMT_MXFP4)                              // the lane holds one 32-channel block per head
#pragma unroll
        for (int m = 0; m < MT; ++m) mx_round_query(C.qa[m]);
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) C.wv[m][r] = a.w[(int64_t)b * a.H_I + 16 * m + 4 * g + r] * a.sigma;
}

// A workgroup's LDS histogram (one word per bin) into its copy of the sequence's.
__device__ __forceinline__ void flush_hist(const uint32_t* hist, uint32_t* hb) {
    flush_hist_copy([&](int i) { return hist[i]; }, hb, hist_copy_of_block(), kScanThreads);
}

// MFMA scan, rows that are not 16-byte multiples (E4M3 132 B, E2M1 72 B).
// Each wave streams chunks of 64 contiguous rows: 16-byte coalesced global loads
// into registers, then into a wave-private LDS stage, from which every lane
// reads the bytes of its MFMA operand.  The next chunk's loads are in flight
// while the current chunk is contracted.  Lane (col = l % 16, g = l / 16) owns
// row col of a 16-row tile and channels g*32 .. g*32+31 (k-slot (g, e) of
// k-step t is channel g*32 + t*8 + e, for A and B alike).
template <int FMT, int MT>
__global__ __launch_bounds__(kScanThreads) void k_scan_staged(ScanArgs a, int rows_per_block) {
    constexpr int RB = idx_rb<FMT>();
    constexpr int kChunkBytes = kChunkRows * RB;
    constexpr int kLoads = (kChunkBytes + 64 * 16 - 1) / (64 * 16);
    __shared__ uint32_t hist[kHistBins];
    __shared__ __attribute__((aligned(16))) uint8_t stage[4][kChunkBytes];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int64_t nvis = clamp_visible(a.n_visible[b], a.capacity);
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_block;
    const int n_chunks = rows_per_block / (4 * kChunkRows);
    for (int i = threadIdx.x; i < kHistBins; i += kScanThreads) hist[i] = 0u;
    ScanCtx<MT> C;
    load_ctx<MT>(C, a, b, col, g);
    __syncthreads();

    const uint8_t* base = a.cache + b * a.stride;
    float* scores = a.scores + b * a.capacity;
    uint8_t* st = stage[wave];
    // chunk c of this wave covers rows row0 + (c * 4 + wave) * 64 ..; two chunks are
    // in flight in two register buffers while the one before them is contracted
    u32x4 rawA[kLoads], rawB[kLoads];
    auto issue = [&](int c, u32x4* raw) {
        const int64_t r = row0 + (int64_t)(c * 4 + wave) * kChunkRows;
        const int64_t avail = (a.capacity - r) * RB;          // bytes of this sequence from r on
        const uint8_t* src = base + r * RB;
        if (avail >= kChunkBytes) {                          // the whole chunk is in the sequence
#pragma unroll
            for (int i = 0; i < kLoads; ++i) {
                const int off = (i * 64 + lane) * 16;
                if (i + 1 < kLoads || off < kChunkBytes)
                    raw[i] = __builtin_bit_cast(u32x4, __builtin_nontemporal_load(
                                                           reinterpret_cast<const u32x4_a4*>(src + off)));
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int off = (i * 64 + lane) * 16;
            raw[i] = u32x4{0u, 0u, 0u, 0u};
            if (off < kChunkBytes && off + 16 <= avail) {
                raw[i] = __builtin_bit_cast(u32x4, __builtin_nontemporal_load(
                                                       reinterpret_cast<const u32x4_a4*>(src + off)));
            } else if (off < kChunkBytes && off < avail) {
                // the sequence ends inside this vector: its last 4, 8 or 12 bytes (rows and
                // strides are multiples of 4 bytes)
                const uint32_t* p = reinterpret_cast<const uint32_t*>(src + off);
                const int n = (int)((avail - off) >> 2);
                raw[i].x = p[0];
                if (n > 1) raw[i].y = p[1];
                if (n > 2) raw[i].z = p[2];
            }
        }
    };
    auto chunk_row = [&](int c) { return row0 + (int64_t)(c * 4 + wave) * kChunkRows; };
    // one chunk: stage its bytes, start the chunk two ahead into the same buffer, contract
    auto step = [&](int c, u32x4* raw) -> bool {
        const int64_t r = chunk_row(c);
        if (r >= a.capacity) return false;
        if (r >= nvis) {                                       // whole chunk masked
            for (int i = lane; i < kChunkRows; i += 64)
                if (r + i < a.capacity) scores[r + i] = -__builtin_inff();
            return true;
        }
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int off = (i * 64 + lane) * 16;
            if (off < kChunkBytes) *reinterpret_cast<u32x4*>(st + off) = raw[i];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (c + 2 < n_chunks && chunk_row(c + 2) < nvis) issue(c + 2, raw);
#pragma unroll
        for (int tile = 0; tile < kChunkRows / 16; ++tile) {
            const int rr = tile * 16 + col;
            const int64_t s = r + rr;
            const bool valid = s < nvis;
            const uint8_t* rp = st + rr * RB;
            uint32_t w[8];
            uint32_t sw = 0;
            float mult = 1.0f;
            if constexpr (FMT == MLA_FMT_E4M3_S128) {
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = reinterpret_cast<const uint32_t*>(rp + g * 32)[i];
                mult = *reinterpret_cast<const float*>(rp + 128);
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = reinterpret_cast<const uint32_t*>(rp + g * 16)[i];
                sw = FMT == MLA_FMT_MXFP4 ? (uint32_t)rp[64 + g] : *reinterpret_cast<const uint16_t*>(rp + 64 + 2 * g);
            }
            u32x4 kb[4];
            dequant_key<FMT>(w, sw, kb);
            if (!valid) mult = 0.0f;
            tile_scores<MT>(C, kb, mult, s, valid, g, a.sigma, a.capacity, scores, hist, a.score_bf16);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        return true;
    };
    if (chunk_row(0) < nvis) issue(0, rawA);
    if (n_chunks > 1 && chunk_row(1) < nvis) issue(1, rawB);
    for (int c = 0; c < n_chunks; c += 2) {
        if (!step(c, rawA)) break;
        if (c + 1 < n_chunks && !step(c + 1, rawB)) break;
    }
    __syncthreads();
    flush_hist(hist, a.hist + (int64_t)b * kHistWordsHost);
}

// Histogram flush of the DMA scans: thread t holds the counts of fine bins
// t + 256 i, so one instruction adds 64 consecutive bins; the coarse counts
// (kept in LDS beside the fine ones) go by the first 64 threads.
template <int NT = kScanThreads>
__device__ __forceinline__ void flush_fine_coarse(const uint32_t (&cnt)[kHistBins / NT], const uint32_t* coarse,
                                                  uint32_t* hb, int copy) {
    uint32_t* fine = hist_fine(hb, copy);
#pragma unroll
    for (int i = 0; i < kHistBins / NT; ++i)
        if (cnt[i]) l2_add(&fine[threadIdx.x + NT * i], cnt[i]);
    if (threadIdx.x < kCoarseBins && coarse[threadIdx.x]) l2_add(&hist_coarse(hb, copy)[threadIdx.x], coarse[threadIdx.x]);
}

// MFMA scan through LDS DMA, E4M3 (132 B) and E2M1 (72 B) rows, for caches
// whose base and sequence stride are 16-byte aligned: a chunk of 32 rows is
// then a 16-byte aligned run of 4224 or 2304 bytes. Each wave streams its own
// chunks (rows row0 + (4 it + wave) * 32 ..) into a private ring of NBUF LDS
// buffers with global_load_lds, without passing them through registers; it
// waits for a chunk with an exact vector-memory count and contracts it as two
// 16-row tiles (operand layout as in k_scan_staged) while the next chunks are
// in flight. The queries and head weights arrive the same way (wave m fetches
// head tile m into its last buffer before that buffer is first used). Scores
// collect in LDS and leave in one coalesced pass; the histogram keeps two
// 16-bit fine bins per word (a block has at most 1024 rows) plus the 64 coarse
// bins, and is flushed by consecutive threads into consecutive bins.
template <int FMT, int MT, int NBUF>
__global__ __launch_bounds__(kScanThreads, kDmaBlocksPerCu) void k_scan_dma(ScanArgs a, int rows_per_block) {
    constexpr int RB = idx_rb<FMT>();
    constexpr int kBytes = kDmaRows * RB;                 // 4224 / 2304
    constexpr int KI = (kBytes + 1023) / 1024;           // DMA instructions per chunk: 5 / 3
    constexpr int kBuf = (KI * 1024 > 5120) ? KI * 1024 : 5120;   // also one head tile of queries + weights
    static_assert(kBytes % 16 == 0, "chunk of 16-byte pieces");
    static_assert(NBUF >= 2 && NBUF <= 3, "ring depth");
    __shared__ uint32_t hist2[kHistBins / 2];
    __shared__ uint32_t coarse[kCoarseBins];
    __shared__ __attribute__((aligned(16))) float sc[kDmaMaxRowsPerBlock];
    __shared__ __attribute__((aligned(16))) uint8_t ring[4][NBUF][kBuf];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, g = lane >> 4;
    const int64_t cap = a.capacity;
    const int64_t nvis = clamp_visible(a.n_visible[b], cap);
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_block;
    const int n_it = rows_per_block / (4 * kDmaRows);
    for (int i = threadIdx.x; i < kHistBins / 2; i += kScanThreads) hist2[i] = 0u;
    if (threadIdx.x < kCoarseBins) coarse[threadIdx.x] = 0u;

    const uint8_t* base = a.cache + b * a.stride;
    auto chunk_row = [&](int it) { return row0 + (int64_t)(4 * it + wave) * kDmaRows; };
    // number of this wave's chunks that start below `lim`
    auto chunks_below = [&](int64_t lim) {
        const int64_t d = lim - row0 - (int64_t)wave * kDmaRows;
        if (d <= 0) return 0;
        const int64_t n = (d + 4 * kDmaRows - 1) / (4 * kDmaRows);
        return (int)(n < n_it ? n : n_it);
    };
    const int n_dma = chunks_below(nvis);                  // chunks with visible rows: read
    const int n_cap = chunks_below(cap);                   // chunks inside the cache: scored
    const uint32_t ring_m0 = __builtin_amdgcn_readfirstlane(lds_addr(&ring[wave][0][0]));
    // KI DMA instructions per chunk, always all of them (the waits count them).
    // Lanes past the chunk, or past the end of the sequence, re-read the
    // chunk's first bytes (cached, never past the cache's end); the rows they
    // stand for are masked.
    auto issue = [&](int it) {
        const int64_t r = chunk_row(it);
        const uint8_t* src = base + r * RB;
        const int64_t left = (cap - r) * RB;
        const uint32_t m0 = ring_m0 + (uint32_t)((it % NBUF) * kBuf);
#pragma unroll
        for (int k = 0; k < KI; ++k) {
            uint32_t off = (uint32_t)(1024 * k + 16 * lane);
            if (off >= (uint32_t)kBytes || (int64_t)off + 16 > left) off = 0;
            dma16_s(src, off, m0 + 1024u * (uint32_t)k);
        }
    };
    // queries of head tile `wave` (16 heads x 128 bf16 = 4 KB) and, by wave 0, the
    // head weights, into the wave's last buffer; then the first chunks
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q_idx) + ((int64_t)b * a.H_I + 16 * wave) * 256;
    if (wave < MT) {
        const uint32_t qm0 = ring_m0 + (uint32_t)((NBUF - 1) * kBuf);
#pragma unroll
        for (int k = 0; k < 4; ++k) dma16_s(qsrc, (uint32_t)(1024 * k + 16 * lane), qm0 + 1024u * (uint32_t)k);
    }
    const float* wstage = reinterpret_cast<const float*>(&ring[0][NBUF - 1][4096]);
    if (wave == 0)
        dma4_s(a.w + (int64_t)b * a.H_I, lane < a.H_I ? 4u * (uint32_t)lane : 0u, ring_m0 + (uint32_t)((NBUF - 1) * kBuf) + 4096u);
    int issued = 0;
    for (; issued < NBUF - 1 && issued < n_dma; ++issued) issue(issued);
    if (NBUF == 3 && issued == 2) wait_vmcnt<2 * KI>();    // the queries have landed
    else if (issued >= 1) wait_vmcnt<KI>();
    else wait_vmcnt<0>();
    if constexpr (FMT == MLA_FMT_MXFP4) {                  // FP4 queries: each wave rounds its staged head tile
        if (wave < MT) {                                   // (lane: head lane / 4, 32-channel block lane % 4)
            uint8_t* hq = &ring[wave][NBUF - 1][0] + (lane >> 2) * 256 + (lane & 3) * 64;
            u32x4 qb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) qb[i] = *reinterpret_cast<const u32x4*>(hq + 16 * i);
            mx_round_query(qb);
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(hq + 16 * i) = qb[i];
        }
    }
    __syncthreads();                                       // queries, weights staged; histograms cleared
    ScanCtx<MT> C;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const uint8_t* qt = &ring[m][NBUF - 1][0];
#pragma unroll
        for (int t = 0; t < 4; ++t) C.qa[m][t] = *reinterpret_cast<const u32x4*>(qt + col * 256 + (g * 32 + t * 8) * 2);
        const f32x4 wv4 = *reinterpret_cast<const f32x4*>(&wstage[16 * m + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) C.wv[m][r] = wv4[r] * a.sigma;
    }
    __syncthreads();                                       // every wave holds them: the buffers are free

    // Software pipeline over the wave's 16-row tiles (two per chunk): the LDS
    // reads and the dequantisation of tile n + 1 are issued between the MFMAs of
    // tile n and its epilogue. Fetching the first tile of chunk c waits for that
    // chunk (the chunks issued after it, c + 1 .. min(c + NBUF - 2, n_dma - 1),
    // may still be in flight) and hands chunk c - 1's buffer, fully read by
    // then, to chunk c + NBUF - 1.
    struct TileIn {
        u32x4 kb[4];
        float mult;
    };
    auto fetch = [&](int c, int tile, TileIn& in) {
        if (tile == 0) {
            if (NBUF == 3 && c + 1 < n_dma) wait_vmcnt<KI>();
            else wait_vmcnt<0>();
            if (c + NBUF - 1 < n_dma) issue(c + NBUF - 1);
        }
        const uint8_t* rp = &ring[wave][c % NBUF][0] + (tile * 16 + col) * RB;
        uint32_t w[8];
        uint32_t sw = 0;
        in.mult = 1.0f;
        if constexpr (FMT == MLA_FMT_E4M3_S128) {
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = reinterpret_cast<const uint32_t*>(rp + g * 32)[i];
            in.mult = *reinterpret_cast<const float*>(rp + 128);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = reinterpret_cast<const uint32_t*>(rp + g * 16)[i];
            sw = FMT == MLA_FMT_MXFP4 ? (uint32_t)rp[64 + g] : *reinterpret_cast<const uint16_t*>(rp + 64 + 2 * g);
        }
        dequant_key<FMT>(w, sw, in.kb);
    };
    const int n_tiles = 2 * n_dma;
    TileIn cur;
    if (n_tiles > 0) fetch(0, 0, cur);
    for (int n = 0; n < n_tiles; ++n) {
        const int c = n >> 1, tile = n & 1;
        f32x4 acc[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = mfma_bf16(C.qa[m][t], cur.kb[t], acc[m]);
        const float mult = cur.mult;
        if (n + 1 < n_tiles) fetch((n + 1) >> 1, (n + 1) & 1, cur);
        const float score = sel_score(tile_epilogue<MT>(C, acc, mult), a.score_bf16);
        const int rr = tile * 16 + col;
        const int lrow = (4 * c + wave) * kDmaRows + rr;   // row within the block
        if (g == tile) {                                   // one lane group per tile writes
            const bool valid = row0 + lrow < nvis;
            sc[lrow] = valid ? score : -__builtin_inff();
            if (valid) {
                const uint32_t bin = score_key(score) >> (32 - kHistBits);
                atomicAdd(&hist2[bin >> 1], 1u << (16 * (bin & 1u)));
                atomicAdd(&coarse[bin / kFinePerCoarse], 1u);
            }
        }
    }
    for (int c = n_dma; c < n_cap; ++c)                     // chunks without a visible row
        if (lane < kDmaRows) sc[(4 * c + wave) * kDmaRows + lane] = -__builtin_inff();
    __syncthreads();
    float* scores = a.scores + b * cap;
    const int64_t nrows = min((int64_t)rows_per_block, cap - row0);
    if (nrows == rows_per_block) {                         // scores + row0 is 512-byte aligned
        for (int i = threadIdx.x; 4 * i < nrows; i += kScanThreads)
            reinterpret_cast<f32x4*>(scores + row0)[i] = reinterpret_cast<const f32x4*>(sc)[i];
    } else {
        for (int i = threadIdx.x; i < nrows; i += kScanThreads) scores[row0 + i] = sc[i];
    }
    // histogram into this XCD's copy: thread t adds fine bins t + 256 i, so one
    // instruction covers 64 consecutive bins
    uint32_t* hb = a.hist + (int64_t)b * kHistWordsHost;
    const int copy = hist_copy_of_block();
    uint32_t cnt[kHistBins / kScanThreads];
#pragma unroll
    for (int i = 0; i < kHistBins / kScanThreads; ++i) {
        const int f = threadIdx.x + kScanThreads * i;
        cnt[i] = (hist2[f >> 1] >> (16 * (f & 1))) & 0xFFFFu;
    }
    flush_fine_coarse(cnt, coarse, hb, copy);
}

// The same scan with the 32x32x16 MFMA, for 32 or 64 indexer heads (MT2 head
// tiles of 32). A 32-row chunk is one tile: lane l owns row l % 32 of the chunk
// and channels 64 (l / 32) .. + 63 (k-step s of the lane is channels
// 64 (l / 32) + 8 s + e, for queries and keys alike), so a row's score is the
// sum over its lane's 16 heads per head tile plus the partner lane's (l ^ 32),
// and the 32 scores of a chunk are written by lanes 0 .. 31 at once.
//
// With FUSE the kernel also carries its step's quantise-append (ap, n_new <=
// kFuseMaxNew entries), cut into pieces of at most 128 channels (piece_load /
// piece_store): wave w of block (x, 0) carries piece 4x + w, loading it as it
// starts, while memory is quiet, and quantising and storing it in registers
// once its own chunks are scored (no LDS, no barrier; extra blocks would
// outgrow the two per CU that run at once), and the wave whose chunk holds a
// new slot stages that entry's fp32 key with
// the queries, quantises it (quant128_wave, byte for byte quant_row's) and
// writes the bytes over the chunk's row in LDS before it dequantises the chunk,
// so the row is scored from the bytes the append writes, whatever the load saw.
// Several queries of one sequence (a shared cache, stride 0: the batch rows are the
// queries): the grid is padded to a multiple of 8 row ranges, and the block index is
// read so that, on each XCD, the G blocks of one row range (one per query) go out
// one after another: they run together and read the range's keys from HBM once,
// the others finding them in that XCD's L2. Blocks past the last range do nothing.
__device__ __forceinline__ bool shared_cache_block(int G, int X, int* bx, int* by) {
    const int L = (int)(blockIdx.y * gridDim.x + blockIdx.x);
    const int j = L >> 3;                                  // the block's place on its XCD (L mod 8)
    *by = j % G;
    *bx = (j / G) * 8 + (L & 7);
    return *bx < X;
}

template <int FMT, int MT2, int NBUF, int NW, bool FUSE>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_scan_dma32(ScanArgs a, int rows_per_block, AppendArgs ap,
                                                                int shared_x) {
    constexpr int NT = 64 * NW;                          // threads of the block
    constexpr int RB = idx_rb<FMT>();
    constexpr int CR = dma32_chunk_rows<FMT>();            // rows per chunk: 32 (E4M3) or 64 (four-bit rows)
    constexpr int TPC = CR / 32;                           // 32-row tiles per chunk
    constexpr int kBytes = CR * RB;                        // 4224 / 4608 / 4352
    constexpr int KI = (kBytes + 1023) / 1024;           // DMA instructions per chunk: 5 / 3
    constexpr int kBuf = (KI * 1024 > 5120) ? KI * 1024 : 5120;   // also one head tile of queries + weights
    static_assert(kBytes % 16 == 0, "chunk of 16-byte pieces");
    static_assert(NBUF >= 2 && NBUF <= 3, "ring depth");
    __shared__ uint32_t hist2[kHistBins / 2];
    __shared__ uint32_t coarse[kCoarseBins];
    __shared__ __attribute__((aligned(16))) float sc[dma32_rows_per_wave<FMT>() * NW];
    __shared__ __attribute__((aligned(16))) uint8_t ring[NW][NBUF][kBuf];
    __shared__ __attribute__((aligned(16))) float fuse_src[FUSE ? kFuseMaxNew : 1][128];
    __shared__ __attribute__((aligned(16))) uint8_t fuse_row[FUSE ? kFuseMaxNew : 1][144];
    static_assert(NW * NBUF * kBuf >= kAppendLdsBytes, "append scratch in the ring");
    int bx = (int)blockIdx.x, b = (int)blockIdx.y;
    if (!FUSE && shared_x > 0 && !shared_cache_block(a.B, shared_x, &bx, &b)) return;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Piece pc;                                              // the carried piece, in registers meanwhile
    if constexpr (FUSE) {
        pc.kind = 0;
        if (b == 0) piece_load(ap, (int64_t)bx * NW + wave, pc);
    }
    const int n32 = lane & 31, h = lane >> 5;
    const int64_t cap = a.capacity;
    const int64_t nvis = clamp_visible(a.n_visible[b], cap);
    const int64_t row0 = (int64_t)bx * rows_per_block;
    // new entries whose slot lies in one of this wave's chunks: own_it[e] is that
    // chunk's iteration (-1: not this wave's), own_r[e] the row in the chunk
    int own_it[FUSE ? kFuseMaxNew : 1], own_r[FUSE ? kFuseMaxNew : 1];
    if constexpr (FUSE) {
#pragma unroll
        for (int e = 0; e < kFuseMaxNew; ++e) {
            own_it[e] = -1;
            own_r[e] = 0;
            if (e < ap.n_new) {
                const int64_t sl = ap.slots[(int64_t)b * ap.n_new + e];
                const int64_t local = sl - row0;
                if (sl >= 0 && sl < cap && local >= 0 && local < rows_per_block) {
                    const int ci = (int)(local / CR);
                    if (ci % NW == wave) {
                        own_it[e] = ci / NW;
                        own_r[e] = (int)(local % CR);
                    }
                }
            }
        }
    }
    const int n_it = rows_per_block / (NW * CR);
    for (int i = threadIdx.x; i < kHistBins / 2; i += NT) hist2[i] = 0u;
    if (threadIdx.x < kCoarseBins) coarse[threadIdx.x] = 0u;

    const uint8_t* base = a.cache + b * a.stride;
    auto chunk_row = [&](int it) { return row0 + (int64_t)(NW * it + wave) * CR; };
    auto chunks_below = [&](int64_t lim) {
        const int64_t d = lim - row0 - (int64_t)wave * CR;
        if (d <= 0) return 0;
        const int64_t n = (d + NW * CR - 1) / (NW * CR);
        return (int)(n < n_it ? n : n_it);
    };
    const int n_dma = chunks_below(nvis);
    const int n_cap = chunks_below(cap);
    const uint32_t ring_m0 = __builtin_amdgcn_readfirstlane(lds_addr(&ring[wave][0][0]));
    // per-lane DMA offsets of a chunk that lies inside the sequence: the lanes
    // past the chunk's bytes re-read its first 16
    uint32_t full_off[KI];
#pragma unroll
    for (int k = 0; k < KI; ++k) {
        const uint32_t o = (uint32_t)(1024 * k + 16 * lane);
        full_off[k] = (o < (uint32_t)kBytes) ? o : 0u;
    }
    auto issue = [&](int it) {
        const int64_t r = chunk_row(it);
        const uint8_t* src = base + r * RB;
        const int64_t left = (cap - r) * RB;
        const uint32_t m0 = ring_m0 + (uint32_t)((it % NBUF) * kBuf);
        if (left >= kBytes) {
#pragma unroll
            for (int k = 0; k < KI; ++k) dma16_s(src, full_off[k], m0 + 1024u * (uint32_t)k);
        } else {                                           // the sequence ends inside the chunk
#pragma unroll
            for (int k = 0; k < KI; ++k) {
                const uint32_t off = ((int64_t)full_off[k] + 16 > left) ? 0u : full_off[k];
                dma16_s(src, off, m0 + 1024u * (uint32_t)k);
            }
        }
    };
    // queries of head tile `wave` (16 heads x 256 B) into the wave's last buffer
    // with a 272-byte head stride (16-byte piece p of head hh at slot 17 hh + p),
    // so that 16 lanes reading one piece of 16 heads hit distinct banks; the head
    // weights (by wave 0) into the score buffer, unused until the chunks start
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q_idx) + ((int64_t)b * a.H_I + 16 * wave) * 256;
    if (wave < 2 * MT2) {
        const uint32_t qm0 = ring_m0 + (uint32_t)((NBUF - 1) * kBuf);
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            const int j = 64 * k + lane, hh = j / 17, pc = j - 17 * hh;
            const uint32_t off = (j < 272 && pc < 16) ? (uint32_t)(256 * hh + 16 * pc) : 0u;
            dma16_s(qsrc, off, qm0 + 1024u * (uint32_t)k);
        }
    }
    const float* wstage = sc;
    if (wave == 0)
        dma4_s(a.w + (int64_t)b * a.H_I, lane < a.H_I ? 4u * (uint32_t)lane : 0u,
               __builtin_amdgcn_readfirstlane(lds_addr(sc)));
    if constexpr (FUSE) {                                  // the owned entries' fp32 keys, 128 channels
#pragma unroll
        for (int e = 0; e < kFuseMaxNew; ++e)
            if (own_it[e] >= 0) {
                const float* src = ap.new_idx + ((int64_t)b * ap.n_new + e) * 128;
                const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(&fuse_src[e][0]));
                dma4_s(src, 4u * (uint32_t)lane, m0);
                dma4_s(src, 256u + 4u * (uint32_t)lane, m0 + 256u);
            }
    }
    int issued = 0;
    for (; issued < NBUF - 1 && issued < n_dma; ++issued) issue(issued);
    if (NBUF == 3 && issued == 2) wait_vmcnt<2 * KI>();
    else if (issued >= 1) wait_vmcnt<KI>();
    else wait_vmcnt<0>();
    if constexpr (FMT == MLA_FMT_MXFP4) {                  // FP4 queries: each wave encodes its staged head tile
        if (wave < 2 * MT2) {                              // (lane: head lane / 4, 32-channel block lane % 4)
            uint8_t* hq = &ring[wave][NBUF - 1][0] + (lane >> 2) * 272 + (lane & 3) * 64;
            u32x4 qb[4], codes;                            // (the block's 16 code bytes, then its scale
#pragma unroll                                             // byte, over the start of its own 64 bytes)
            for (int i = 0; i < 4; ++i) qb[i] = *reinterpret_cast<const u32x4*>(hq + 16 * i);
            const uint32_t e8 = mx_encode_query(qb, codes);
            *reinterpret_cast<u32x4*>(hq) = codes;
            *reinterpret_cast<uint32_t*>(hq + 16) = e8;
        }
    }
    __syncthreads();                                       // queries, weights staged; histograms cleared
    if constexpr (FUSE) {
#pragma unroll
        for (int e = 0; e < kFuseMaxNew; ++e)
            if (own_it[e] >= 0)
                quant128_wave<FMT>(fuse_src[e][2 * lane], fuse_src[e][2 * lane + 1], &fuse_row[e][0],
                                   &fuse_row[e][FMT == MLA_FMT_E4M3_S128 ? 128 : 64]);
    }
    u32x4 qa[MT2][8];                                      // head 32 mt + n32, channels 64 h + 8 s ..
    uint32_t qsc[MT2];                                     // MXFP4: scales of blocks 2h, 2h + 1; E2M1: the head's k
    float wv[MT2][16];                                     // w * sigma of result register v
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt) {
        const int head = 32 * mt + n32;
        const uint8_t* qt = &ring[head >> 4][NBUF - 1][0] + (head & 15) * 272 + 128 * h;
        if constexpr (FMT == MLA_FMT_MXFP4) {
            qa[mt][0] = *reinterpret_cast<const u32x4*>(qt);
            qa[mt][1] = *reinterpret_cast<const u32x4*>(qt + 64);
            qsc[mt] = (*reinterpret_cast<const uint32_t*>(qt + 16) & 0xFFu) |
                      ((*reinterpret_cast<const uint32_t*>(qt + 80) & 0xFFu) << 8);
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s) qa[mt][s] = *reinterpret_cast<const u32x4*>(qt + 16 * s);
        }
        if constexpr (FMT == MLA_FMT_E2M1_S16) {           // fp16 operands: the head scaled by 2^k into range
            uint32_t m = 0;
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    m = max(m, max((qa[mt][s][e] << 16) & 0x7FFFFFFFu, qa[mt][s][e] & 0x7FFF0000u));
            m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
            const int k = min(max(14 - ((int)(m >> 23) - 127), -120), 120);
            qsc[mt] = (uint32_t)k;
#pragma unroll
            for (int s = 0; s < 8; ++s) qa[mt][s] = bf16x8_to_f16x8_scaled(qa[mt][s], u2f((uint32_t)(k + 127) << 23));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(&wstage[32 * mt + 8 * q + 4 * h]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                wv[mt][4 * q + r] = w4[r] * a.sigma;
                if constexpr (FMT == MLA_FMT_E2M1_S16)      // the row's head was scaled by 2^k: undo it
                    wv[mt][4 * q + r] *= u2f((uint32_t)(127 - __shfl((int)qsc[mt], 8 * q + 4 * h + r, 64)) << 23);
            }
        }
    }
    __syncthreads();                                       // every wave holds them: the buffers are free

    // the codes of chunk c, dequantised: k-step s of this lane (waits for the
    // chunk and hands chunk c - 1's buffer to chunk c + NBUF - 1 first)
    struct ChunkIn {
        u32x4 kb[8];
        float mult;
        uint32_t ks;                                       // MXFP4: the E8M0 codes of blocks 2h, 2h + 1
    };
    // (tile t of chunk t / TPC: the chunk's wait, its successor's issue and the
    // new entries' rows happen at its first tile)
    auto fetch = [&](int t, ChunkIn& in) {
        const int c = t / TPC;
        if (t % TPC == 0) {
            if (NBUF == 3 && c + 1 < n_dma) wait_vmcnt<KI>();
            else wait_vmcnt<0>();
            if (c + NBUF - 1 < n_dma) issue(c + NBUF - 1);
            if constexpr (FUSE) {                          // a new entry's row: its bytes over the stale ones
#pragma unroll
                for (int e = 0; e < kFuseMaxNew; ++e)
                    if (own_it[e] == c && lane < RB / 4)
                        reinterpret_cast<uint32_t*>(&ring[wave][c % NBUF][0] + own_r[e] * RB)[lane] =
                            reinterpret_cast<const uint32_t*>(&fuse_row[e][0])[lane];
            }
        }
        const uint8_t* rp = &ring[wave][c % NBUF][0] + ((t % TPC) * 32 + n32) * RB;
        in.mult = 1.0f;
        if constexpr (FMT == MLA_FMT_E4M3_S128) {
            uint32_t w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = reinterpret_cast<const uint32_t*>(rp + 64 * h)[i];
            in.mult = *reinterpret_cast<const float*>(rp + 128);
            dequant_key<FMT>(w, 0u, in.kb);
            dequant_key<FMT>(w + 8, 0u, in.kb + 4);
        } else {
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = reinterpret_cast<const uint32_t*>(rp + 32 * h)[i];
            if constexpr (FMT == MLA_FMT_MXFP4) {               // the codes as they are, for the FP4 MFMA
                in.kb[0] = u32x4{w[0], w[1], w[2], w[3]};
                in.kb[1] = u32x4{w[4], w[5], w[6], w[7]};
                in.ks = *reinterpret_cast<const uint16_t*>(rp + 64 + 2 * h);
            } else {
                const uint32_t sw = *reinterpret_cast<const uint32_t*>(rp + 64 + 4 * h);
                dequant_e2m1_f16(w, sw & 0xFFFFu, in.kb);
                dequant_e2m1_f16(w + 4, sw >> 16, in.kb + 4);
            }
        }
    };
    ChunkIn cur;
    const int n_tiles = TPC * n_dma;
    if (n_tiles > 0) fetch(0, cur);
    for (int tt = 0; tt < n_tiles; ++tt) {
        f32x16 acc[MT2];
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mt][v] = 0.0f;
        }
        if constexpr (FMT == MLA_FMT_MXFP4) {              // FP4 x FP4 with the blocks' E8M0 scales
#pragma unroll
            for (int mt = 0; mt < MT2; ++mt) {
                acc[mt] = mfma32_fp4(qa[mt][0], cur.kb[0], acc[mt], qsc[mt] & 0xFFu, cur.ks & 0xFFu);
                acc[mt] = mfma32_fp4(qa[mt][1], cur.kb[1], acc[mt], qsc[mt] >> 8, cur.ks >> 8);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 8; ++s)
#pragma unroll
                for (int mt = 0; mt < MT2; ++mt)
                    acc[mt] = FMT == MLA_FMT_E2M1_S16 ? mfma32_f16(qa[mt][s], cur.kb[s], acc[mt])
                                                      : mfma32_bf16(qa[mt][s], cur.kb[s], acc[mt]);
        }
        const float mult = cur.mult;
        if (tt + 1 < n_tiles) fetch(tt + 1, cur);
        // sum_j w_j ReLU(sigma * mult * d_j) = mult * sum_j (w_j sigma) ReLU(d_j)  (sigma, mult >= 0)
        float pm[MT2][4];
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                pm[mt][q] = wv[mt][4 * q] * relu(acc[mt][4 * q]);
#pragma unroll
                for (int r = 1; r < 4; ++r) pm[mt][q] += wv[mt][4 * q + r] * relu(acc[mt][4 * q + r]);
            }
        float part = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt) part += (pm[mt][0] + pm[mt][1]) + (pm[mt][2] + pm[mt][3]);
        const float score = sel_score(xsum2(part) * mult, a.score_bf16);
        const int lrow = (NW * (tt / TPC) + wave) * CR + (tt % TPC) * 32 + n32;  // row within the block
        if (h == 0) {
            const bool valid = row0 + lrow < nvis;
            sc[lrow] = valid ? score : -__builtin_inff();
            if (valid) {
                const uint32_t bin = score_key(score) >> (32 - kHistBits);
                atomicAdd(&hist2[bin >> 1], 1u << (16 * (bin & 1u)));
                atomicAdd(&coarse[bin / kFinePerCoarse], 1u);
            }
        }
    }
    if constexpr (FUSE) piece_store(ap, pc);               // every load of the wave has landed
    for (int c = n_dma; c < n_cap; ++c)                     // chunks without a visible row
        if (lane < CR) sc[(NW * c + wave) * CR + lane] = -__builtin_inff();
    __syncthreads();
    float* scores = a.scores + b * cap;
    const int64_t nrows = min((int64_t)rows_per_block, cap - row0);
    if (nrows == rows_per_block) {
        for (int i = threadIdx.x; 4 * i < nrows; i += NT)
            reinterpret_cast<f32x4*>(scores + row0)[i] = reinterpret_cast<const f32x4*>(sc)[i];
    } else {
        for (int i = threadIdx.x; i < nrows; i += NT) scores[row0 + i] = sc[i];
    }
    uint32_t* hb = a.hist + (int64_t)b * kHistWordsHost;
    const int copy = hist_copy_of_block();
    uint32_t cnt[kHistBins / NT];
#pragma unroll
    for (int i = 0; i < kHistBins / NT; ++i) {
        const int f = threadIdx.x + NT * i;
        cnt[i] = (hist2[f >> 1] >> (16 * (f & 1))) & 0xFFFFu;
    }
    flush_fine_coarse<NT>(cnt, coarse, hb, copy);

}

// The 32x32 scan with its chunks handed out at run time. Workgroup (x, y)
// serves queue x as its member y (gridDim.x queues, 2^lg_groups per sequence,
// gridDim.y workgroups each; workgroups go out x-fastest, one member of every
// queue before the next); index arithmetic is shifts and masks only, so the
// first loads leave at once.
// queue (b, g) owns the 32-row chunks [g n / groups, (g + 1) n / groups) of
// sequence b's n visible chunks. Each wave of the queue's W = per_queue * NW
// waves takes its first kScanStaticJobs chunks by its index (x W + wq past the
// queue's first, job x), then one chunk per ticket drawn from the queue's
// counter: the ticket for the wave's job j + 2 is drawn when job j is issued,
// two jobs ahead of its use, so waves that are served early take more chunks
// and all finish together. No ticket is drawn before the wave's first chunks
// have landed: at the start every wave would draw at once and the atomics on
// one counter are served one after another. The
// tickets, the chunk loads and the score stores of a wave complete in issue
// order, and every wait counts exactly the operations issued after the one it
// needs. The last wave of a queue to finish returns its counters to zero.
// The histogram is kept with one 32-bit word per fine bin (a workgroup may see
// any number of rows); the scores of a chunk are stored by lanes 0 .. 31.
template <int FMT, int MT2, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void k_scan_dyn32(ScanArgs a, int lg_groups) {
    constexpr int NBUF = 3;
    constexpr int NT = 64 * NW;
    constexpr int RB = idx_rb<FMT>();
    constexpr int kBytes = kDmaRows * RB;                 // 4224 / 2304
    constexpr int KI = (kBytes + 1023) / 1024;           // DMA instructions per chunk: 5 / 3
    constexpr int kBuf = (KI * 1024 > 5120) ? KI * 1024 : 5120;   // also one head tile of queries
    constexpr int S = kScanStaticJobs;
    static_assert(kBytes % 16 == 0, "chunk of 16-byte pieces");
    static_assert(S >= 2 && S <= 4, "static jobs: a ticket is drawn with jobs S - 2 ..");
    __shared__ uint32_t hist[kHistBins];
    __shared__ uint32_t coarse[kCoarseBins];
    __shared__ __attribute__((aligned(16))) float wst[64];
    __shared__ __attribute__((aligned(16))) uint8_t ring[NW][NBUF][kBuf];
    const int qi = blockIdx.x, member = blockIdx.y, per_queue = gridDim.y;
    const int groups = 1 << lg_groups;
    const int b = qi >> lg_groups, g = qi & (groups - 1);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n32 = lane & 31, h = lane >> 5;
    const int64_t cap = a.capacity;
    const int64_t nvis = clamp_visible(a.n_visible[b], cap);
    const int64_t nch = (nvis + kDmaRows - 1) >> 5;                // chunks holding visible rows
    const int64_t c_lo = (nch * g) >> lg_groups, c_hi = (nch * (g + 1)) >> lg_groups;
    const int64_t W = (int64_t)per_queue * NW;
    const int64_t wq = (int64_t)member * NW + wave;
    uint32_t* const qctr = a.queues + kQueueWordsHost * qi;
    for (int i = threadIdx.x; i < kHistBins; i += NT) hist[i] = 0u;
    if (threadIdx.x < kCoarseBins) coarse[threadIdx.x] = 0u;

    const uint8_t* base = a.cache + b * a.stride;
    const uint32_t ring_m0 = __builtin_amdgcn_readfirstlane(lds_addr(&ring[wave][0][0]));
    uint32_t full_off[KI];
#pragma unroll
    for (int k = 0; k < KI; ++k) {
        const uint32_t o = (uint32_t)(1024 * k + 16 * lane);
        full_off[k] = (o < (uint32_t)kBytes) ? o : 0u;
    }
    auto issue = [&](int64_t ch, int slot) {               // chunk ch into ring slot `slot`: KI loads
        const int64_t r = ch * kDmaRows;
        const uint8_t* src = base + r * RB;
        const int64_t left = (cap - r) * RB;
        const uint32_t m0 = ring_m0 + (uint32_t)(slot * kBuf);
        if (left >= kBytes) {
#pragma unroll
            for (int k = 0; k < KI; ++k) dma16_s(src, full_off[k], m0 + 1024u * (uint32_t)k);
        } else {                                           // the sequence ends inside the chunk
#pragma unroll
            for (int k = 0; k < KI; ++k) {
                const uint32_t off = ((int64_t)full_off[k] + 16 > left) ? 0u : full_off[k];
                dma16_s(src, off, m0 + 1024u * (uint32_t)k);
            }
        }
    };
    // wait until at most n operations are in flight (n: a count this kernel produces)
    auto wait_upto = [&](int n) {
        if (n >= KI + 3) wait_vmcnt_asm<KI + 3>();
        else if (n == KI + 2) wait_vmcnt_asm<KI + 2>();
        else if (n == KI + 1) wait_vmcnt_asm<KI + 1>();
        else if (n == KI) wait_vmcnt_asm<KI>();
        else if (n >= 2) wait_vmcnt_asm<2>();
        else if (n == 1) wait_vmcnt_asm<1>();
        else wait_vmcnt_asm<0>();
    };

    // job x: a static chunk for x < S, else the chunk of a ticket drawn with job x - 2
    auto static_chunk = [&](int x) { return c_lo + (int64_t)x * W + wq; };
    auto ticket_chunk = [&](uint32_t t) { return c_lo + (int64_t)S * W + (int64_t)t; };
    // ---- prologue: queries and weights, job 0, job 1 (each with its ticket if S = 2, 3)
    const int64_t ch0 = static_chunk(0), ch1 = static_chunk(1);
    const bool v0 = ch0 < c_hi, v1 = ch1 < c_hi;
    uint32_t tA = 0u, tB = 0u;                             // tickets in flight: drawn with even jobs in tA, odd in tB
    const uint8_t* qsrc = reinterpret_cast<const uint8_t*>(a.q_idx) + ((int64_t)b * a.H_I + 16 * wave) * 256;
    if (wave < 2 * MT2) {                                  // head tile `wave`, 272-byte head stride
        const uint32_t qm0 = ring_m0 + (uint32_t)((NBUF - 1) * kBuf);
#pragma unroll
        for (int k = 0; k < 5; ++k) {
            const int j = 64 * k + lane, hh = j / 17, pc = j - 17 * hh;
            const uint32_t off = (j < 272 && pc < 16) ? (uint32_t)(256 * hh + 16 * pc) : 0u;
            dma16_s(qsrc, off, qm0 + 1024u * (uint32_t)k);
        }
    }
    if (wave == 0)
        dma4_s(a.w + (int64_t)b * a.H_I, lane < a.H_I ? 4u * (uint32_t)lane : 0u,
               __builtin_amdgcn_readfirstlane(lds_addr(wst)));
    if (v0) {
        if (S <= 2) ticket_issue(tA, qctr);
        issue(ch0, 0);
    }
    if (v1) {
        if (S <= 3) ticket_issue(tB, qctr);
        issue(ch1, 1);
    }
    if (v1) {                                              // all but job 1 (and its ticket)
        if (S <= 3) wait_vmcnt_asm<KI + 1>();
        else wait_vmcnt_asm<KI>();
    } else {
        wait_vmcnt_asm<0>();
    }
    if constexpr (FMT == MLA_FMT_MXFP4) {                  // FP4 queries: each wave rounds its staged head tile
        if (wave < 2 * MT2) {                              // (lane: head lane / 4, 32-channel block lane % 4)
            uint8_t* hq = &ring[wave][NBUF - 1][0] + (lane >> 2) * 272 + (lane & 3) * 64;
            u32x4 qb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) qb[i] = *reinterpret_cast<const u32x4*>(hq + 16 * i);
            mx_round_query(qb);
#pragma unroll
            for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(hq + 16 * i) = qb[i];
        }
    }
    __syncthreads();                                       // queries, weights staged; histograms cleared
    u32x4 qa[MT2][8];
    float wv[MT2][16];
#pragma unroll
    for (int mt = 0; mt < MT2; ++mt) {
        const int head = 32 * mt + n32;
        const uint8_t* qt = &ring[head >> 4][NBUF - 1][0] + (head & 15) * 272 + 128 * h;
#pragma unroll
        for (int s = 0; s < 8; ++s) qa[mt][s] = *reinterpret_cast<const u32x4*>(qt + 16 * s);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(&wst[32 * mt + 8 * q + 4 * h]);
#pragma unroll
            for (int r = 0; r < 4; ++r) wv[mt][4 * q + r] = w4[r] * a.sigma;
        }
    }
    __syncthreads();                                       // every wave holds them: the buffers are free

    struct ChunkIn {
        u32x4 kb[8];
        float mult;
    };
    auto dequant = [&](int slot, ChunkIn& in) {
        const uint8_t* rp = &ring[wave][slot][0] + n32 * RB;
        in.mult = 1.0f;
        if constexpr (FMT == MLA_FMT_E4M3_S128) {
            uint32_t w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = reinterpret_cast<const uint32_t*>(rp + 64 * h)[i];
            in.mult = *reinterpret_cast<const float*>(rp + 128);
            dequant_key<FMT>(w, 0u, in.kb);
            dequant_key<FMT>(w + 8, 0u, in.kb + 4);
        } else {
            uint32_t w[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) w[i] = reinterpret_cast<const uint32_t*>(rp + 32 * h)[i];
            if constexpr (FMT == MLA_FMT_MXFP4) {
                const uint32_t sw = *reinterpret_cast<const uint16_t*>(rp + 64 + 2 * h);
                dequant_key<FMT>(w, sw & 0xFFu, in.kb);
                dequant_key<FMT>(w + 4, sw >> 8, in.kb + 4);
            } else {
                const uint32_t sw = *reinterpret_cast<const uint32_t*>(rp + 64 + 4 * h);
                dequant_key<FMT>(w, sw & 0xFFFFu, in.kb);
                dequant_key<FMT>(w + 4, sw >> 16, in.kb + 4);
            }
        }
    };

    // jobs: the current job j (chunk chj), then jobs j + 1 and j + 2 (chunk, valid)
    ChunkIn cur;
    int64_t chj = ch0, chn1 = ch1, chn2 = 0;
    bool vn1 = v1, vn2 = false;
    if (v0) {                                              // job 0 landed: issue job 2
        const int64_t c2 = (S > 2) ? static_chunk(2) : ticket_chunk(ticket_read(tA));
        vn2 = c2 < c_hi;
        chn2 = c2;
        if (vn2) {
            ticket_issue(tA, qctr);                        // ticket for job 4
            issue(c2, 2);
        }
        dequant(0, cur);
    }
    float* scores = a.scores + b * cap;
    // job j on `cur`; treg holds the ticket drawn with job j + 1 (the one for job j + 3)
    auto step = [&](int j, uint32_t& treg) -> bool {
        f32x16 acc[MT2];
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[mt][v] = 0.0f;
        }
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int mt = 0; mt < MT2; ++mt) acc[mt] = mfma32_bf16(qa[mt][s], cur.kb[s], acc[mt]);
        const float mult = cur.mult;
        const int64_t row = chj * kDmaRows + n32;
        const bool more = vn1;
        if (vn1) {
            // in flight after job j + 1's loads: the score store of job j - 2, job j + 2's
            // ticket (drawn from job S - 2 on) and loads, the score store of job j - 1
            wait_upto((j >= 2 ? 1 : 0) + (vn2 ? KI + (j + 2 >= S - 2 ? 1 : 0) : 0) + (j >= 1 ? 1 : 0));
            const int64_t c3 = (j + 3 < S) ? static_chunk(j + 3) : ticket_chunk(ticket_read(treg));
            const bool v3 = c3 < c_hi;
            if (v3) {
                ticket_issue(treg, qctr);                  // ticket for job j + 5
                issue(c3, (j + 3) % 3);                    // into job j's slot, already read
            }
            dequant((j + 1) % 3, cur);
            chj = chn1;
            chn1 = chn2;
            vn1 = vn2;
            chn2 = c3;
            vn2 = v3;
        }
        // sum_j w_j ReLU(sigma * mult * d_j) = mult * sum_j (w_j sigma) ReLU(d_j)  (sigma, mult >= 0)
        float pm[MT2][4];
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                pm[mt][q] = wv[mt][4 * q] * relu(acc[mt][4 * q]);
#pragma unroll
                for (int r = 1; r < 4; ++r) pm[mt][q] += wv[mt][4 * q + r] * relu(acc[mt][4 * q + r]);
            }
        float part = 0.0f;
#pragma unroll
        for (int mt = 0; mt < MT2; ++mt) part += (pm[mt][0] + pm[mt][1]) + (pm[mt][2] + pm[mt][3]);
        const float score = sel_score(xsum2(part) * mult, a.score_bf16);
        if (h == 0 && row < cap) {                         // row 0 of the chunk is visible: one store
            const bool valid = row < nvis;
            scores[row] = valid ? score : -__builtin_inff();
            if (valid) {
                const uint32_t bin = score_key(score) >> (32 - kHistBits);
                atomicAdd(&hist[bin], 1u);
                atomicAdd(&coarse[bin / kFinePerCoarse], 1u);
            }
        }
        return more;
    };
    if (v0) {
        for (int j = 0;; j += 2) {
            if (!step(j, tB)) break;
            if (!step(j + 1, tA)) break;
        }
    }
    wait_vmcnt<0>();
    // finished: count the wave out of its queue (the reply is read after the flush)
    uint32_t fin = 0u;
    if (lane == 0) fin = __hip_atomic_fetch_add(qctr + 16, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // rows past the visible chunks: -inf, strided over the workgroups of the sequence
    {
        const int64_t stride = (int64_t)groups * per_queue * NT;
        for (int64_t r = nch * kDmaRows + ((int64_t)g * per_queue + member) * NT + threadIdx.x; r < cap; r += stride)
            scores[r] = -__builtin_inff();
    }
    __syncthreads();
    uint32_t* hb = a.hist + (int64_t)b * kHistWordsHost;
    uint32_t cnt[kHistBins / NT];
#pragma unroll
    for (int i = 0; i < kHistBins / NT; ++i) cnt[i] = hist[threadIdx.x + NT * i];
    flush_fine_coarse<NT>(cnt, coarse, hb, hist_copy_of_block());
    if (lane == 0 && fin == (uint32_t)W - 1) {             // the queue's last wave: counters back to zero
        __hip_atomic_store(qctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(qctr + 16, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// MFMA scan, 256-byte bf16 rows (16-byte aligned): direct 16-byte loads.
// bf16 indexer keys (256-byte rows): each wave contracts 16-row tiles loaded straight
// into its B operands, the next tile's loads issued before the current tile is
// contracted; the queries are staged once per workgroup in LDS.
// With FUSE the kernel also carries its step's append (ap, at most kFuseMaxNew entries
// per sequence) as the 32x32 scan does: wave w of block (x, 0) loads piece 4 x + w
// as it starts and stores it after its tiles, and a row that is one of the new slots
// is scored from the new key rounded to bf16 (staged in LDS), the bytes the append
// writes, whatever its load saw.
template <int MT, bool FUSE>
__global__ __launch_bounds__(kScanThreads) void k_scan_bf16(ScanArgs a, int rows_per_block, AppendArgs ap) {
    __shared__ uint32_t hist[kHistBins];
    __shared__ __attribute__((aligned(16))) uint16_t new_key[FUSE ? kFuseMaxNew : 1][128];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    Piece pc;                                              // the carried piece, in registers meanwhile
    if constexpr (FUSE) {
        pc.kind = 0;
        if (b == 0) piece_load(ap, (int64_t)blockIdx.x * 4 + wave, pc);
    }
    const int64_t nvis = clamp_visible(a.n_visible[b], a.capacity);
    const int64_t row0 = (int64_t)blockIdx.x * rows_per_block;
    const int n_it = rows_per_block / 64;                  // 16-row tiles per wave
    const uint8_t* base = a.cache + b * a.stride;
    float* scores = a.scores + b * a.capacity;
    // the tile's B operands (zero past the visible rows); the next tile's loads are issued
    // before the current tile is contracted
    auto load_tile = [&](int it, u32x4* kb) {
        const int64_t s = row0 + (int64_t)(it * 4 + wave) * 16 + col;
        if (s < nvis) {
            const u32x4* p = reinterpret_cast<const u32x4*>(base + s * 256 + g * 64);
#pragma unroll
            for (int t = 0; t < 4; ++t) kb[t] = __builtin_nontemporal_load(p + t);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) kb[t] = u32x4{0u, 0u, 0u, 0u};
        }
    };
    // the sequence's queries staged once per workgroup (272-byte head stride: the 16 lanes
    // reading one piece of 16 heads hit distinct banks), then read into every wave's operands
    __shared__ __attribute__((aligned(16))) uint8_t qs[16 * MT * 272];
    u32x4 kb[4], kn[4];
    load_tile(0, kb);
    {
        const uint8_t* qb = reinterpret_cast<const uint8_t*>(a.q_idx) + (int64_t)b * a.H_I * 256;
        for (int i = threadIdx.x; i < 16 * MT * 16; i += kScanThreads)
            *reinterpret_cast<u32x4*>(qs + (i >> 4) * 272 + 16 * (i & 15)) =
                *reinterpret_cast<const u32x4*>(qb + 16 * i);
    }
    int64_t slot[FUSE ? kFuseMaxNew : 1];                  // the new slots of the sequence (-1: none)
    if constexpr (FUSE) {
#pragma unroll
        for (int e = 0; e < kFuseMaxNew; ++e) {
            slot[e] = -1;
            if (e < ap.n_new) {
                const int64_t sl = ap.slots[(int64_t)b * ap.n_new + e];
                if (sl >= 0 && sl < a.capacity) slot[e] = sl;
            }
        }
        const int e = threadIdx.x >> 6;                    // wave e stages new key e, 2 channels per lane
        if (e < ap.n_new) {
            const f32x2 v = *reinterpret_cast<const f32x2*>(ap.new_idx + ((int64_t)b * ap.n_new + e) * 128 + 2 * lane);
            reinterpret_cast<uint32_t*>(&new_key[e][0])[lane] = bf16_rne(v.x) | (bf16_rne(v.y) << 16);
        }
    }
    for (int i = threadIdx.x; i < kHistBins; i += kScanThreads) hist[i] = 0u;
    ScanCtx<MT> C;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) C.wv[m][r] = a.w[(int64_t)b * a.H_I + 16 * m + 4 * g + r] * a.sigma;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            C.qa[m][t] = *reinterpret_cast<const u32x4*>(qs + (16 * m + col) * 272 + 2 * (g * 32 + t * 8));
    for (int it = 0; it < n_it; ++it) {
        const int64_t tile0 = row0 + (int64_t)(it * 4 + wave) * 16;
        if (tile0 >= a.capacity) break;
        if (it + 1 < n_it) load_tile(it + 1, kn);
        const int64_t s = tile0 + col;
        const bool valid = s < nvis;
        if constexpr (FUSE) {                              // a new slot's row: the new key's bytes
#pragma unroll
            for (int e = 0; e < kFuseMaxNew; ++e)
                if (s == slot[e]) {
#pragma unroll
                    for (int t = 0; t < 4; ++t)
                        kb[t] = valid ? *reinterpret_cast<const u32x4*>(&new_key[e][g * 32 + t * 8])
                                      : u32x4{0u, 0u, 0u, 0u};
                }
        }
        if (tile0 >= nvis) {
            if (g == 0 && s < a.capacity) scores[s] = -__builtin_inff();
        } else {
            tile_scores<MT>(C, kb, valid ? 1.0f : 0.0f, s, valid, g, a.sigma, a.capacity, scores, hist,
                            a.score_bf16);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) kb[t] = kn[t];
    }
    if constexpr (FUSE) piece_store(ap, pc);
    __syncthreads();
    flush_hist(hist, a.hist + (int64_t)b * kHistWordsHost);
}

// MFMA scan of a candidate pool ([P4] "The Hierarchical Sparse
// Indexer: bounded sweeps"; [P1] "DeepSeek-V4.1", "The hierarchical indexer": a Reindex layer scores only the positions a
// Full layer published). Entry i of sequence b is the row at position
// cand[b, i]; its score goes to scores[b, i] (-inf when the position is
// negative or not visible) and every entry, -inf ones included, is counted in
// the histogram, so that the selection can treat the pool as n_cand visible
// entries. The pool is small (16384 rows of 72 B at V4.1's sizes), so the
// kernel is built for latency: each lane loads the bytes of its own MFMA
// operand straight from the row (rows of a pool are scattered, and only
// 4-byte (E4M3), 8-byte (E2M1) or 16-byte (bf16) aligned), all of a wave's
// loads are issued before the first contraction, and each workgroup takes
// kCandTiles 16-entry tiles per wave. Lane (col, g) owns entry col of a tile
// and channels g*32 .. g*32+31, as in the streaming scans.
constexpr int kCandTiles = 2;
template <int FMT, int MT>
__global__ __launch_bounds__(kScanThreads) void k_scan_cand(ScanArgs a) {
    __shared__ uint32_t hist[kHistBins];
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int64_t nvis = clamp_visible(a.n_visible[b], a.capacity);
    const int64_t n = a.n_cand;
    const int32_t* cand = a.cand + b * n;
    const uint8_t* base = a.cache + b * a.stride;
    float* scores = a.scores + b * n;
    int64_t ent[kCandTiles];
    bool valid[kCandTiles];
    int32_t pos[kCandTiles];
#pragma unroll
    for (int t = 0; t < kCandTiles; ++t) {
        ent[t] = ((int64_t)blockIdx.x * 4 * kCandTiles + t * 4 + wave) * 16 + col;
        pos[t] = ent[t] < n ? cand[ent[t]] : -1;
    }
    // the row loads: E4M3 8 words of codes + the fp32 scale, E2M1 4 words of
    // nibbles + the two scale bytes of the lane's channels (MXFP4: one byte),
    // bf16 four 16-byte vectors
    constexpr int NW = (FMT == MLA_FMT_E4M3_S128) ? 8 : (FMT == MLA_FMT_BF16 ? 16 : 4);
    uint32_t w[kCandTiles][NW];
    uint32_t sw[kCandTiles];
#pragma unroll
    for (int t = 0; t < kCandTiles; ++t) {
        valid[t] = pos[t] >= 0 && pos[t] < nvis;
        const uint8_t* row = base + (int64_t)(valid[t] ? pos[t] : 0) * a.row_bytes;
        if constexpr (FMT == MLA_FMT_E4M3_S128) {
            const uint32_t* p = reinterpret_cast<const uint32_t*>(row + g * 32);
#pragma unroll
            for (int i = 0; i < 8; ++i) w[t][i] = valid[t] ? p[i] : 0u;
            sw[t] = valid[t] ? *reinterpret_cast<const uint32_t*>(row + 128) : 0u;
        } else if constexpr (FMT == MLA_FMT_E2M1_S16) {
            const u32x2* p = reinterpret_cast<const u32x2*>(row + g * 16);
            const u32x2 lo = valid[t] ? p[0] : u32x2{0u, 0u}, hi = valid[t] ? p[1] : u32x2{0u, 0u};
            w[t][0] = lo.x;
            w[t][1] = lo.y;
            w[t][2] = hi.x;
            w[t][3] = hi.y;
            sw[t] = valid[t] ? *reinterpret_cast<const uint16_t*>(row + 64 + 2 * g) : 0u;
        } else if constexpr (FMT == MLA_FMT_MXFP4) {          // 68-byte rows: 4-byte aligned
            const uint32_t* p = reinterpret_cast<const uint32_t*>(row + g * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) w[t][i] = valid[t] ? p[i] : 0u;
            sw[t] = valid[t] ? (uint32_t)row[64 + g] : 0u;
        } else {
            const u32x4* p = reinterpret_cast<const u32x4*>(row + g * 64);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x4 x = valid[t] ? p[i] : u32x4{0u, 0u, 0u, 0u};
                w[t][4 * i] = x.x;
                w[t][4 * i + 1] = x.y;
                w[t][4 * i + 2] = x.z;
                w[t][4 * i + 3] = x.w;
            }
            sw[t] = 0u;
        }
    }
    ScanCtx<MT> C;
    load_ctx<MT>(C, a, b, col, g);
    for (int i = threadIdx.x; i < kHistBins; i += kScanThreads) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int t = 0; t < kCandTiles; ++t) {
        u32x4 kb[4];
        float mult = valid[t] ? 1.0f : 0.0f;
        if constexpr (FMT == MLA_FMT_BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) kb[i] = u32x4{w[t][4 * i], w[t][4 * i + 1], w[t][4 * i + 2], w[t][4 * i + 3]};
        } else {
            dequant_key<FMT>(w[t], sw[t], kb);
            if constexpr (FMT == MLA_FMT_E4M3_S128) mult = valid[t] ? __builtin_bit_cast(float, sw[t]) : 0.0f;
        }
        const float part = sel_score(tile_dot<MT>(C, kb, mult), a.score_bf16);
        if (g == 0 && ent[t] < n) {
            const float sc = valid[t] ? part : -__builtin_inff();
            scores[ent[t]] = sc;
            atomicAdd(&hist[score_key(sc) >> (32 - kHistBits)], 1u);
        }
    }
    __syncthreads();
    flush_hist(hist, a.hist + (int64_t)b * kHistWordsHost);
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
    case MLA_FMT_MXFP4: {
        const uint32_t byte = row[c / 2];
        return e2m1_value((c & 1) ? (byte >> 4) : (byte & 15u)) * e8m0_to_f32(row[dim / 2 + c / 32]);
    }
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
    if (a.fmt == MLA_FMT_MXFP4) {                             // FP4 queries: each 32-channel block rounded
        __syncthreads();
        for (int blk = threadIdx.x; blk < n / 32; blk += kScanThreads) {
            uint32_t m = 0;
            for (int c = 0; c < 32; ++c) m = max(m, f2u(fabsf(qs[32 * blk + c])));
            const uint32_t code = mx_code(m);
            for (int c = 0; c < 32; ++c) {
                const uint32_t nib = mx_encode(qs[32 * blk + c], m, code);
                qs[32 * blk + c] = e2m1_value(nib) * e8m0_to_f32(code);
            }
        }
    }
    for (int i = threadIdx.x; i < kHistBins; i += kScanThreads) hist[i] = 0u;
    __syncthreads();
    // entry s: row s, or with a candidate pool the row at position cand[b, s]
    // (every pool entry is counted in the histogram, -inf ones included)
    const int64_t n_out = a.cand ? a.n_cand : a.capacity;
    const int64_t s = (int64_t)blockIdx.x * kScanThreads + threadIdx.x;
    const int64_t nvis = clamp_visible(a.n_visible[b], a.capacity);
    if (s < n_out) {
        const int64_t pos = a.cand ? (int64_t)a.cand[b * n_out + s] : s;
        float score = -__builtin_inff();
        if (pos >= 0 && pos < nvis) {
            const uint8_t* row = a.cache + b * a.stride + pos * a.row_bytes;
            score = 0.0f;
            for (int j = 0; j < a.H_I; ++j) {
                float d = 0.0f;
                for (int c = 0; c < a.dim; ++c) d += qs[j * a.dim + c] * key_elem(a.fmt, a.dim, row, c);
                score += a.w[(int64_t)b * a.H_I + j] * fmaxf(a.sigma * d, 0.0f);
            }
        }
        score = sel_score(score, a.score_bf16);
        if (a.cand || pos < nvis) atomicAdd(&hist[score_key(score) >> (32 - kHistBits)], 1u);
        a.scores[b * n_out + s] = score;
    }
    __syncthreads();
    flush_hist(hist, a.hist + (int64_t)b * kHistWordsHost);
}

}  // namespace

bool scan_supported(int fmt, int dim, int H_I) {
    if (H_I <= 0) return false;
    if ((fmt == MLA_FMT_BF16 || fmt == MLA_FMT_E4M3_S128 || fmt == MLA_FMT_E2M1_S16 || fmt == MLA_FMT_MXFP4) &&
        dim == 128 &&
        H_I % 16 == 0 && H_I <= 64)
        return true;
    return H_I * dim <= 8192;
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream, const AppendArgs* append) {
    // the step's append rides in the 32x32 scan's launch when that kernel runs and the
    // append writes the scanned cache; otherwise it is launched on its own, first
    const bool carry = append && append->n_new >= 1 && append->n_new <= kFuseMaxNew && append->B == a.B &&
                       append->idx_cache == a.cache && append->idx_stride == a.stride && a.dim == 128;
    auto unfused = [&]() -> hipError_t {
        if (append) {
            const hipError_t e = launch_append(*append, stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    };
    const bool mfma = (a.fmt == MLA_FMT_BF16 || a.fmt == MLA_FMT_E4M3_S128 || a.fmt == MLA_FMT_E2M1_S16 ||
                       a.fmt == MLA_FMT_MXFP4) &&
                      a.dim == 128 && a.H_I % 16 == 0 && a.H_I <= 64;
    if (a.cand) {                                              // a candidate pool: n_cand entries per sequence
        if (const hipError_t e = unfused(); e != hipSuccess) return e;
        if (a.B == 0 || a.n_cand == 0) return hipSuccess;
        const ProfSlot p = prof_slot(PROF_SCAN);
        if (mfma) {
            const dim3 grid((unsigned)((a.n_cand + 64 * kCandTiles - 1) / (64 * kCandTiles)), a.B);
#define MLA_CAND_CASE(F, M)                                                                    \
    if (a.fmt == F && a.H_I == 16 * M)                                                         \
        return launch_kernel(k_scan_cand<F, M>, grid, dim3(kScanThreads), 0, stream, p.start, p.stop, a);
            MLA_CAND_CASE(MLA_FMT_BF16, 1) MLA_CAND_CASE(MLA_FMT_BF16, 2)
            MLA_CAND_CASE(MLA_FMT_BF16, 3) MLA_CAND_CASE(MLA_FMT_BF16, 4)
            MLA_CAND_CASE(MLA_FMT_E4M3_S128, 1) MLA_CAND_CASE(MLA_FMT_E4M3_S128, 2)
            MLA_CAND_CASE(MLA_FMT_E4M3_S128, 3) MLA_CAND_CASE(MLA_FMT_E4M3_S128, 4)
            MLA_CAND_CASE(MLA_FMT_E2M1_S16, 1) MLA_CAND_CASE(MLA_FMT_E2M1_S16, 2)
            MLA_CAND_CASE(MLA_FMT_E2M1_S16, 3) MLA_CAND_CASE(MLA_FMT_E2M1_S16, 4)
            MLA_CAND_CASE(MLA_FMT_MXFP4, 1) MLA_CAND_CASE(MLA_FMT_MXFP4, 2)
            MLA_CAND_CASE(MLA_FMT_MXFP4, 3) MLA_CAND_CASE(MLA_FMT_MXFP4, 4)
#undef MLA_CAND_CASE
            return hipErrorInvalidValue;
        }
        const dim3 grid((unsigned)((a.n_cand + kScanThreads - 1) / kScanThreads), a.B);
        return launch_kernel(k_scan_generic, grid, dim3(kScanThreads), 0, stream, p.start, p.stop, a);
    }
    if (a.B == 0 || a.capacity == 0) return unfused();
    if (mfma) {
        // bf16 keys: rows per block (a multiple of 64, at most kRowsPerBlock) for about one
        // block per CU, so that short caches still fill the chip (c2, 8 x 8192 rows: 256
        // blocks measured 0.3 us per step ahead of 384, 512 and 768)
        int64_t bblocks = 256;
        if (const int64_t v = option(OPT_SCAN_BLOCKS)) bblocks = v;
        const int64_t bper_seq = std::max<int64_t>(1, bblocks / a.B);
        int64_t brpb = (a.capacity + bper_seq - 1) / bper_seq;
        brpb = std::min<int64_t>(std::max<int64_t>((brpb + 63) / 64 * 64, 64), kRowsPerBlock);
        const dim3 bgrid((unsigned)((a.capacity + brpb - 1) / brpb), a.B);
        // staged scan: ~kStagedBlocks long-lived workgroups, each wave streaming many chunks
        const int64_t per_seq = (kStagedBlocks + a.B - 1) / a.B;
        int64_t rpb = (a.capacity + per_seq - 1) / per_seq;
        rpb = ((rpb + 4 * kChunkRows - 1) / (4 * kChunkRows)) * (4 * kChunkRows);
        const dim3 sgrid((unsigned)((a.capacity + rpb - 1) / rpb), a.B);
        // LDS-DMA scan: 16-byte aligned cache and stride; about kDmaBlocksPerCu blocks per CU
        // (and a sequence's rows end on a 16-byte boundary: the chunk that holds the last
        // row loads whole 16-byte pieces up to the sequence's end, none beyond it)
        const bool dma = (reinterpret_cast<uintptr_t>(a.cache) % 16 == 0) && (a.stride % 16 == 0) &&
                         (a.capacity * a.row_bytes) % 16 == 0;
        // the scan_blocks option overrides the target number of blocks (for tuning)
        int64_t dma_target = 256 * kDmaBlocksPerCu;
        if (const int64_t v = option(OPT_SCAN_BLOCKS)) dma_target = v;
        const int64_t dma_per_seq = (dma_target + a.B - 1) / a.B;
        int64_t drpb = (a.capacity + dma_per_seq - 1) / dma_per_seq;
        drpb = ((drpb + 4 * kDmaRows - 1) / (4 * kDmaRows)) * (4 * kDmaRows);
        drpb = std::min<int64_t>(std::max<int64_t>(drpb, 4 * kDmaRows), kDmaMaxRowsPerBlock);
        const dim3 dgrid((unsigned)((a.capacity + drpb - 1) / drpb), a.B);
        // the 32x32 scan: blocks of kDma32Waves waves, as many as the CUs hold at once
        // (two 4-wave blocks per CU, whatever the ring depth)
        int64_t blk32 = 256 * (8 / kDma32Waves);
        if (const int64_t v = option(OPT_SCAN_BLOCKS)) blk32 = std::max<int64_t>(1, v * 4 / kDma32Waves);
        const int64_t per_seq32 = (blk32 + a.B - 1) / a.B;
        const int64_t unit32 = (int64_t)kDma32Waves * (a.fmt == MLA_FMT_E4M3_S128 ? kDmaRows : 2 * kDmaRows);
        int64_t d32rpb = (a.capacity + per_seq32 - 1) / per_seq32;
        d32rpb = ((d32rpb + unit32 - 1) / unit32) * unit32;
        const int64_t rpw32 = a.fmt == MLA_FMT_E4M3_S128 ? kDmaRowsPerWave : kDmaRowsPerWave4;
        d32rpb = std::min<int64_t>(std::max<int64_t>(d32rpb, unit32), rpw32 * kDma32Waves);
        const dim3 d32grid((unsigned)((a.capacity + d32rpb - 1) / d32rpb), a.B);
        // several queries of one shared cache: row ranges padded to a multiple of 8 (see
        // shared_cache_block), the same rows per block as for one sequence
        const bool shared = a.stride == 0 && a.B > 1 && !carry;
        const dim3 d32grid_sh((d32grid.x + 7) / 8 * 8, a.B);
        // the queue-fed 32x32 scan (option scan_queues; at the T = 128K shape it is
        // slower than the static partition): about 64 queues (a sequence's rows
        // split into `groups` ranges), 2 blocks per CU in all, at least about 4
        // chunks per wave
        const bool dyn = a.queues != nullptr && a.B <= kScanQueuesHost && option(OPT_SCAN_QUEUES) != 0;
        int dyn_lg = 0;
        while (a.B << (dyn_lg + 1) <= 64) ++dyn_lg;            // 2^lg queues per sequence, B 2^lg <= 64
        const int64_t dyn_nq = (int64_t)a.B << dyn_lg;
        const int64_t dyn_chunks = (int64_t)a.B * ((a.capacity + kDmaRows - 1) / kDmaRows);
        const int64_t dyn_per_queue = std::max<int64_t>(
            1, std::min<int64_t>(blk32 / dyn_nq, dyn_chunks / (dyn_nq * kDma32Waves * 4)));
#define MLA_SCAN_CASE(F, M)                                                                    \
    if (a.fmt == F && a.H_I == 16 * M) {                                                       \
        if constexpr (F == MLA_FMT_BF16) {                                                     \
            if (carry && pieces_supported(*append) && piece_count(*append) <= (int64_t)bgrid.x * 4) { \
                const ProfSlot p = prof_slot(PROF_SCAN);                                       \
                return launch_kernel(k_scan_bf16<M, true>, bgrid, dim3(kScanThreads), 0, stream, p.start, \
                                     p.stop, a, (int)brpb, *append);                           \
            }                                                                                  \
            if (const hipError_t e = unfused(); e != hipSuccess) return e;                     \
            const ProfSlot p = prof_slot(PROF_SCAN);                                           \
            return launch_kernel(k_scan_bf16<M, false>, bgrid, dim3(kScanThreads), 0, stream, p.start, p.stop, a, \
                                 (int)brpb, AppendArgs{});                                     \
        } else {                                                                               \
            const ProfSlot p = prof_slot(PROF_SCAN);                                           \
            if (dma) {                                                                         \
                if constexpr (M % 2 == 0) {                                                    \
                    if (!dyn && carry && pieces_supported(*append) &&                          \
                        piece_count(*append) <= (int64_t)d32grid.x * kDma32Waves)              \
                        return launch_kernel(k_scan_dma32<F, M / 2, F == MLA_FMT_E4M3_S128 ? kDmaNbuf : kDmaNbuf4, kDma32Waves, true>,    \
                                             d32grid, dim3(64 * kDma32Waves), 0, stream, p.start, p.stop, \
                                             a, (int)d32rpb, *append, 0);                      \
                    if (const hipError_t e = unfused(); e != hipSuccess) return e;             \
                    if (dyn)                                                                   \
                        return launch_kernel(k_scan_dyn32<F, M / 2, kDma32Waves>,              \
                                             dim3((unsigned)dyn_nq, (unsigned)dyn_per_queue), dim3(64 * kDma32Waves), \
                                             0, stream, p.start, p.stop, a, dyn_lg);   \
                    return launch_kernel(k_scan_dma32<F, M / 2, F == MLA_FMT_E4M3_S128 ? kDmaNbuf : kDmaNbuf4, kDma32Waves, false>, \
                                         shared ? d32grid_sh : d32grid, dim3(64 * kDma32Waves), 0, stream, p.start, \
                                         p.stop, a, (int)d32rpb, AppendArgs{}, shared ? (int)d32grid.x : 0); \
                }                                                                              \
                else {                                                                         \
                    if (const hipError_t e = unfused(); e != hipSuccess) return e;             \
                    return launch_kernel(k_scan_dma<F, M, kDmaNbuf>, dgrid, dim3(kScanThreads), 0, \
                                         stream, p.start, p.stop, a, (int)drpb);               \
                }                                                                              \
            }                                                                                  \
            if (const hipError_t e = unfused(); e != hipSuccess) return e;                     \
            return launch_kernel(k_scan_staged<F, M>, sgrid, dim3(kScanThreads), 0, stream, p.start, p.stop, \
                                 a, (int)rpb);                                                 \
        }                                                                                      \
    }
        MLA_SCAN_CASE(MLA_FMT_BF16, 1) MLA_SCAN_CASE(MLA_FMT_BF16, 2)
        MLA_SCAN_CASE(MLA_FMT_BF16, 3) MLA_SCAN_CASE(MLA_FMT_BF16, 4)
        MLA_SCAN_CASE(MLA_FMT_E4M3_S128, 1) MLA_SCAN_CASE(MLA_FMT_E4M3_S128, 2)
        MLA_SCAN_CASE(MLA_FMT_E4M3_S128, 3) MLA_SCAN_CASE(MLA_FMT_E4M3_S128, 4)
        MLA_SCAN_CASE(MLA_FMT_E2M1_S16, 1) MLA_SCAN_CASE(MLA_FMT_E2M1_S16, 2)
        MLA_SCAN_CASE(MLA_FMT_E2M1_S16, 3) MLA_SCAN_CASE(MLA_FMT_E2M1_S16, 4)
        MLA_SCAN_CASE(MLA_FMT_MXFP4, 1) MLA_SCAN_CASE(MLA_FMT_MXFP4, 2)
        MLA_SCAN_CASE(MLA_FMT_MXFP4, 3) MLA_SCAN_CASE(MLA_FMT_MXFP4, 4)
#undef MLA_SCAN_CASE
        return hipErrorInvalidValue;
    }
    if (const hipError_t e = unfused(); e != hipSuccess) return e;
    const dim3 grid((unsigned)((a.capacity + kScanThreads - 1) / kScanThreads), a.B);
    const ProfSlot p = prof_slot(PROF_SCAN);
    return launch_kernel(k_scan_generic, grid, dim3(kScanThreads), 0, stream, p.start, p.stop, a);
}

}  // namespace mla
