// decode.hip -- absorbed-MLA sparse decode: shared-KV MQA over the selected
// latent entries plus the window, softmax, logsumexp output.
//
// For each (b, h), over U = {selected rows} + {window slots}:
//   z_u = scale * q[b,h,:] . K_u,  lse = logsumexp z,  out = sum_u e^(z_u - lse) K_u[:d_v]
// ([P1] "DeepSeek's Attention and KV Cache - From MLA to CSA2", "DeepSeek-V2",
// "Why RoPE breaks the trick" and "Check it in numpy"; [P2] "From MLA to DSA
// to HCA/CSA", Part 2 "What replaced MLA"; each selected latent is read once
// for all heads, [P1] "DeepSeek-V3.2", "The lightning indexer").
//
// MFMA path (H a multiple of 16 up to 128, d_v = 512, K width 576 = 512 + 64 or 512):
//   grid (splits, B, head groups); a split is `rps` <= 128 consecutive entries of
//   idx[b] (or of the window ring); workgroup = 4 waves that all gather, and the
//   first NHT = min(4, H / 16) of them also contract: wave w owns heads
//   16 * (NHT * blockIdx.z + w) .. +15, whose queries sit in LDS.
//   Two phases over the split's 32-row chunks, the next chunk's row bytes always
//   loaded into registers while the current one is contracted:
//   * QK phase: the workgroup dequantises each chunk's rows exactly into a bf16
//     row-major K tile (E4M3 codes unscaled, E2M1 x scale); each wave computes
//     S^T = K q^T on bf16 MFMA (E4M3: one accumulator per 128-channel block times
//     the row's fp32 scale) and keeps the split's scores in registers.  The exact
//     per-head maximum and sum of exponentials follow, so no rescaling is ever
//     needed and the fp32 output tile is only touched by the MFMA.
//   * PV phase: the rows are read again (now from L2) into a channel-major V^T
//     tile (fp16: E4M3 codes / E2M1 x scale are exact in fp16; bf16 for bf16
//     rows), and O^T = V^T P^T accumulates on MFMA with fp16 P (E4M3: P times the
//     row's scale over the split's largest scale of that block, <= 1) or bf16 P
//     split into a high and a low part when V is bf16.
//   The split's normalised output and logsumexp are written as a partial and
//   k_merge combines the partials by logsumexp.
// Generic path (any other shape): one workgroup per (b, h), fp32 on the vector
// ALUs, writes the final output directly.
#include <cstdlib>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kChunk = 32;
constexpr int kMaxChunks = 4;             // rows per split <= 128
constexpr int kDv = 512;
constexpr int kVt = 36;                   // halves per V^T channel (32 rows + pad)
constexpr int kVtGroupPad = 32;           // halves after every 32 channels: spreads LDS banks
constexpr int kVtSize = kDv * kVt + (kDv / 32) * kVtGroupPad;
constexpr int kMergeThreads = kDv / 4;
constexpr int kGenericThreads = 256;
constexpr int kGenericMaxRows = 8192;

enum SrcKind { SRC_E4M3 = 0, SRC_FP4 = 1, SRC_BF16 = 2 };

__device__ __forceinline__ int vt_off(int c) { return c * kVt + (c >> 5) * kVtGroupPad; }

// Entries per split (a multiple of 32, at most 128): fewer splits mean fewer
// fp32 partials to write and merge, more splits more workgroups in flight.
// MLA_DECODE_RPS overrides the default for tuning; the workspace query reads it too.
int rows_per_split(int H, int k) {
    if (const char* e = getenv("MLA_DECODE_RPS")) {
        const int v = atoi(e);
        if (v >= 32 && v <= 32 * kMaxChunks && v % 32 == 0) return v;
    }
    (void)H;
    (void)k;
    return 64;
}

template <int DQK>
struct Lds {
    static constexpr int kKs = DQK + 8;                  // bf16 per K / q row (padded)
    static constexpr int kTile = (kChunk * kKs > kVtSize) ? kChunk * kKs : kVtSize;
    uint16_t qs[64 * kKs];                               // queries of the workgroup's heads
    uint16_t tile[kTile];                                // QK phase: K rows; PV phase: V^T
    float fac[kChunk][4];                                // E4M3 row scales (QK) / scale over split max (PV)
    int32_t valid[kChunk];
    uint32_t smax_bits[4];                               // E4M3: the split's largest row scale per block
    float inv_smax[4];                                   // E4M3: 1 / smax (1 where the block has no row)
};

// Raw bytes of one QK-phase item (32 channels of one row).
struct SlotA {
    u32x4 v[4];
    uint32_t x;           // E4M3: the scale word of the segment's block; E2M1: two scale bytes
    int ok;
};
// Raw bytes of one PV-phase item (32 value channels of a pair of rows).
struct SlotB {
    u32x4 v[2][4];
    uint32_t x[2];
    int ok[2];
};

template <int SRC>
__device__ __forceinline__ void load_a(SlotA& sl, const uint8_t* __restrict__ row, int sg) {
    if constexpr (SRC == SRC_BF16) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + sg * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) sl.v[i] = p[i];
    } else if constexpr (SRC == SRC_E4M3) {
        if (sg < 16) {
            const u32x4* p = reinterpret_cast<const u32x4*>(row + sg * 32);
            sl.v[0] = p[0];
            sl.v[1] = p[1];
            sl.x = reinterpret_cast<const uint32_t*>(row + 512)[sg >> 2];
        } else {  // bf16 RoPE channels 512 + 32 (sg - 16) ..
            const u32x4* p = reinterpret_cast<const u32x4*>(row + 528 + (sg - 16) * 64);
#pragma unroll
            for (int i = 0; i < 4; ++i) sl.v[i] = p[i];
        }
    } else {  // SRC_FP4: 16 nibble bytes + 2 scale bytes per 32 channels
        sl.v[0] = *reinterpret_cast<const u32x4*>(row + sg * 16);
        sl.x = *reinterpret_cast<const uint16_t*>(row + 256 + 2 * sg);
    }
}

template <int SRC>
__device__ __forceinline__ void load_b(SlotB& sl, int h, const uint8_t* __restrict__ row, int sg) {
    if constexpr (SRC == SRC_BF16) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + sg * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) sl.v[h][i] = p[i];
    } else if constexpr (SRC == SRC_E4M3) {
        const u32x4* p = reinterpret_cast<const u32x4*>(row + sg * 32);
        sl.v[h][0] = p[0];
        sl.v[h][1] = p[1];
        sl.x[h] = reinterpret_cast<const uint32_t*>(row + 512)[sg >> 2];
    } else {
        sl.v[h][0] = *reinterpret_cast<const u32x4*>(row + sg * 16);
        sl.x[h] = *reinterpret_cast<const uint16_t*>(row + 256 + 2 * sg);
    }
}

// 32 values of segment sg of a PV-phase item row: fp16 (E4M3 / E2M1, exact) or bf16 bits.
template <int SRC>
__device__ __forceinline__ void value_bits(const SlotB& sl, int h, uint16_t out[32]) {
    if constexpr (SRC == SRC_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                out[8 * i + 2 * e] = (uint16_t)(sl.v[h][i][e] & 0xFFFFu);
                out[8 * i + 2 * e + 1] = (uint16_t)(sl.v[h][i][e] >> 16);
            }
    } else if constexpr (SRC == SRC_E4M3) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t w = sl.v[h][i >> 2][i & 3];
            const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
            const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true));
            out[4 * i] = (uint16_t)(lo & 0xFFFFu);
            out[4 * i + 1] = (uint16_t)(lo >> 16);
            out[4 * i + 2] = (uint16_t)(hi & 0xFFFFu);
            out[4 * i + 3] = (uint16_t)(hi >> 16);
        }
    } else {
        const float s0 = e4m3_to_f32(sl.x[h] & 0xFFu), s1 = e4m3_to_f32((sl.x[h] >> 8) & 0xFFu);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sc = (i < 2) ? s0 : s1;
            const uint32_t w = sl.v[h][0][i];
            const f32x2 v[4] = {e2m1x2_to_f32<0>(w), e2m1x2_to_f32<1>(w), e2m1x2_to_f32<2>(w), e2m1x2_to_f32<3>(w)};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                out[8 * i + 2 * e] = __builtin_bit_cast(uint16_t, (_Float16)(v[e].x * sc));
                out[8 * i + 2 * e + 1] = __builtin_bit_cast(uint16_t, (_Float16)(v[e].y * sc));
            }
        }
    }
}

__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// One split: QK phase, exact softmax statistics, PV phase, partial.
template <int SRC, int DQK, int NHT>
__device__ __forceinline__ void decode_split(const DecodeArgs& a, Lds<DQK>& L, int b, int split, int S,
                                             bool is_win, int64_t first, int n_rows, float* o_part,
                                             float* lse_part) {
    constexpr int NT = DQK / 32;           // k-steps of QK = 32-channel segments of a K row
    constexpr int NTH = 256;               // every wave loads; waves w < NHT also contract
    constexpr int NITEM_A = kChunk * NT;
    constexpr int NSLOT_A = (NITEM_A + NTH - 1) / NTH;
    constexpr int NITEM_B = (kChunk / 2) * (kDv / 32);   // (row pair, value segment)
    constexpr int NSLOT_B = (NITEM_B + NTH - 1) / NTH;
    constexpr int KS = Lds<DQK>::kKs;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    const bool mw = w < NHT;
    const int head = 16 * (NHT * (int)blockIdx.z + w) + j;
    constexpr float kLog2e = 1.4426950408889634f;
    const float zscale = a.scale * kLog2e;
    const int nc = (n_rows + kChunk - 1) / kChunk;

    auto row_ptr = [&](int u) -> const uint8_t* {
        if (u >= n_rows) return nullptr;
        if (is_win) return reinterpret_cast<const uint8_t*>(a.win + ((int64_t)b * a.W + first + u) * DQK);
        const int32_t s = a.idx[(int64_t)b * a.k + first + u];
        if (s < 0 || s >= a.capacity) return nullptr;
        return a.cache + b * a.stride + (int64_t)s * a.row_bytes;
    };
    auto load_chunk_a = [&](int c0, SlotA* sl) {
#pragma unroll
        for (int i = 0; i < NSLOT_A; ++i) {
            const int item = tid + i * NTH;
            sl[i].ok = 0;
            if (item < NITEM_A) {
                const uint8_t* rp = row_ptr(c0 + item % kChunk);
                if (rp) {
                    sl[i].ok = 1;
                    load_a<SRC>(sl[i], rp, item / kChunk);
                }
            }
        }
    };
    auto load_chunk_b = [&](int c0, SlotB* sl) {
#pragma unroll
        for (int i = 0; i < NSLOT_B; ++i) {
            const int item = tid + i * NTH;
            sl[i].ok[0] = sl[i].ok[1] = 0;
            if (item < NITEM_B) {
                const int rp = item % (kChunk / 2), sg = item / (kChunk / 2);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint8_t* p = row_ptr(c0 + 2 * rp + h);
                    if (p) {
                        sl[i].ok[h] = 1;
                        load_b<SRC>(sl[i], h, p, sg);
                    }
                }
            }
        }
    };
    auto store_chunk_a = [&](const SlotA* sl) {
#pragma unroll
        for (int i = 0; i < NSLOT_A; ++i) {
            const int item = tid + i * NTH;
            if (item >= NITEM_A) continue;
            const int sg = item / kChunk, r = item % kChunk;
            uint32_t* kd = reinterpret_cast<uint32_t*>(L.tile + r * KS + sg * 32);
            if (!sl[i].ok) {
#pragma unroll
                for (int q = 0; q < 4; ++q) reinterpret_cast<u32x4*>(kd)[q] = u32x4{0u, 0u, 0u, 0u};
                if (SRC == SRC_E4M3 && sg < 4) L.fac[r][sg] = 0.0f;
            } else if constexpr (SRC == SRC_BF16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) reinterpret_cast<u32x4*>(kd)[q] = sl[i].v[q];
            } else if constexpr (SRC == SRC_E4M3) {
                if (sg < 16) {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        const u32x2 p0 = e4m3x4_to_bf16(sl[i].v[q].x), p1 = e4m3x4_to_bf16(sl[i].v[q].y);
                        const u32x2 p2 = e4m3x4_to_bf16(sl[i].v[q].z), p3 = e4m3x4_to_bf16(sl[i].v[q].w);
                        reinterpret_cast<u32x4*>(kd)[2 * q] = u32x4{p0.x, p0.y, p1.x, p1.y};
                        reinterpret_cast<u32x4*>(kd)[2 * q + 1] = u32x4{p2.x, p2.y, p3.x, p3.y};
                    }
                    if ((sg & 3) == 0) {
                        L.fac[r][sg >> 2] = u2f(sl[i].x);
                        atomicMax(&L.smax_bits[sg >> 2], sl[i].x);     // positive fp32 orders as uint
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 4; ++q) reinterpret_cast<u32x4*>(kd)[q] = sl[i].v[q];
                }
            } else {  // E2M1 x E4M3 scale, exact in bf16
                const float s0 = e4m3_to_f32(sl[i].x & 0xFFu), s1 = e4m3_to_f32((sl[i].x >> 8) & 0xFFu);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float sc = (q < 2) ? s0 : s1;
                    const uint32_t wv = sl[i].v[0][q];
                    const f32x2 v0 = e2m1x2_to_f32<0>(wv), v1 = e2m1x2_to_f32<1>(wv);
                    const f32x2 v2 = e2m1x2_to_f32<2>(wv), v3 = e2m1x2_to_f32<3>(wv);
                    reinterpret_cast<u32x4*>(kd)[q] =
                        u32x4{pack_bf16_trunc(v0.x * sc, v0.y * sc), pack_bf16_trunc(v1.x * sc, v1.y * sc),
                              pack_bf16_trunc(v2.x * sc, v2.y * sc), pack_bf16_trunc(v3.x * sc, v3.y * sc)};
                }
            }
            if (sg == 0) L.valid[r] = sl[i].ok;
        }
    };
    auto store_chunk_b = [&](const SlotB* sl) {
#pragma unroll
        for (int i = 0; i < NSLOT_B; ++i) {
            const int item = tid + i * NTH;
            if (item >= NITEM_B) continue;
            const int rp = item % (kChunk / 2), sg = item / (kChunk / 2);
            uint16_t v0[32], v1[32];
            if (sl[i].ok[0]) value_bits<SRC>(sl[i], 0, v0);
            else {
#pragma unroll
                for (int e = 0; e < 32; ++e) v0[e] = 0;
            }
            if (sl[i].ok[1]) value_bits<SRC>(sl[i], 1, v1);
            else {
#pragma unroll
                for (int e = 0; e < 32; ++e) v1[e] = 0;
            }
#pragma unroll
            for (int e = 0; e < 32; ++e)
                *reinterpret_cast<uint32_t*>(L.tile + vt_off(sg * 32 + e) + 2 * rp) =
                    (uint32_t)v0[e] | ((uint32_t)v1[e] << 16);
            if (SRC == SRC_E4M3 && (sg & 3) == 0) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    L.fac[2 * rp + h][sg >> 2] = sl[i].ok[h] ? u2f(sl[i].x[h]) * L.inv_smax[sg >> 2] : 0.0f;
            }
        }
    };

    // ---- start the first chunk's loads, then stage the queries
    SlotA sa[NSLOT_A];
    SlotB sb[NSLOT_B];
    if (nc > 0) load_chunk_a(0, sa);
    {
        constexpr int NQ = 16 * NHT * (DQK / 8);           // 16-byte pieces of the queries
        constexpr int NQT = (NQ + NTH - 1) / NTH;
        const int head0 = 16 * NHT * (int)blockIdx.z;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.H + head0) * DQK;
        u32x4 qv[NQT];
#pragma unroll
        for (int i = 0; i < NQT; ++i) {
            const int e = tid + i * NTH;
            if (e < NQ) qv[i] = *reinterpret_cast<const u32x4*>(qp + (int64_t)(e / (DQK / 8)) * DQK + (e % (DQK / 8)) * 8);
        }
#pragma unroll
        for (int i = 0; i < NQT; ++i) {
            const int e = tid + i * NTH;
            if (e < NQ) *reinterpret_cast<u32x4*>(L.qs + (e / (DQK / 8)) * KS + (e % (DQK / 8)) * 8) = qv[i];
        }
        if (tid < 4) L.smax_bits[tid] = 0u;
    }
    const uint16_t* qrow = L.qs + (16 * w + j) * KS + g * 8;

    // ---- QK phase: scores of all chunks into registers (base 2, scaled)
    float z[kMaxChunks][2][4];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) z[c][rt][r] = -__builtin_inff();
        if (c >= nc) continue;
        __syncthreads();                                   // previous tile fully consumed (and q staged)
        store_chunk_a(sa);
        __syncthreads();
        if (c + 1 < nc) load_chunk_a((c + 1) * kChunk, sa);
        else load_chunk_b(0, sb);                          // PV phase's first chunk, in flight now
        if (!mw) continue;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const uint16_t* ka = L.tile + (16 * rt + j) * KS + g * 8;
            f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (SRC == SRC_E4M3) {
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4) {
                    f32x4 t4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 4 * b4; t < 4 * b4 + 4; ++t)
                        t4 = mfma_bf16(*reinterpret_cast<const u32x4*>(ka + t * 32),
                                       *reinterpret_cast<const u32x4*>(qrow + t * 32), t4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) sacc[r] += t4[r] * L.fac[16 * rt + 4 * g + r][b4];
                }
#pragma unroll
                for (int t = 16; t < NT; ++t)
                    sacc = mfma_bf16(*reinterpret_cast<const u32x4*>(ka + t * 32),
                                     *reinterpret_cast<const u32x4*>(qrow + t * 32), sacc);
            } else {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    sacc = mfma_bf16(*reinterpret_cast<const u32x4*>(ka + t * 32),
                                     *reinterpret_cast<const u32x4*>(qrow + t * 32), sacc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (L.valid[16 * rt + 4 * g + r]) z[c][rt][r] = sacc[r] * zscale;
        }
    }

    // ---- exact softmax statistics of the split, per head (lanes j, j+16, j+32, j+48)
    float m = -__builtin_inff();
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, z[c][rt][r]);
    m = fmaxf(m, __shfl_xor(m, 16, 64));
    m = fmaxf(m, __shfl_xor(m, 32, 64));
    float l = 0.0f;
    if (m != -__builtin_inff()) {
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    z[c][rt][r] = __builtin_amdgcn_exp2f(z[c][rt][r] - m);     // exp2(-inf) = 0
                    l += z[c][rt][r];
                }
    } else {                                               // no visible entry: P = 0, never -inf
#pragma unroll
        for (int c = 0; c < kMaxChunks; ++c)
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) z[c][rt][r] = 0.0f;
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if constexpr (SRC == SRC_E4M3) {
        __syncthreads();                                   // every row's scale is in smax_bits
        if (tid < 4) {                                     // read by the PV stores after their barrier
            const float sm = u2f(L.smax_bits[tid]);
            L.inv_smax[tid] = (sm > 0.0f) ? 1.0f / sm : 1.0f;
        }
    }

    // ---- PV phase: O^T += V^T P^T; k-slot (g, e): e < 4 -> row 4g+e, e >= 4 -> row 16+4g+e-4
    f32x4 oacc[kDv / 16];
#pragma unroll
    for (int i = 0; i < kDv / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        if (c >= nc) continue;
        __syncthreads();
        store_chunk_b(sb);
        __syncthreads();
        if (c + 1 < nc) load_chunk_b((c + 1) * kChunk, sb);
        if (!mw) continue;
        const float (*p)[4] = z[c];
        if constexpr (SRC == SRC_BF16) {
            float hi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = p[e >> 2][e & 3];
                hi[e] = u2f(bf16_rne(v) << 16);
                lo[e] = v - hi[e];
            }
            const u32x4 ph = u32x4{bf16_rne(hi[0]) | (bf16_rne(hi[1]) << 16), bf16_rne(hi[2]) | (bf16_rne(hi[3]) << 16),
                                   bf16_rne(hi[4]) | (bf16_rne(hi[5]) << 16), bf16_rne(hi[6]) | (bf16_rne(hi[7]) << 16)};
            const u32x4 pl = u32x4{bf16_rne(lo[0]) | (bf16_rne(lo[1]) << 16), bf16_rne(lo[2]) | (bf16_rne(lo[3]) << 16),
                                   bf16_rne(lo[4]) | (bf16_rne(lo[5]) << 16), bf16_rne(lo[6]) | (bf16_rne(lo[7]) << 16)};
#pragma unroll
            for (int mt = 0; mt < kDv / 16; ++mt) {
                const uint16_t* va = L.tile + vt_off(16 * mt + j);
                const u32x2 x0 = *reinterpret_cast<const u32x2*>(va + 4 * g);
                const u32x2 x1 = *reinterpret_cast<const u32x2*>(va + 16 + 4 * g);
                const u32x4 av = u32x4{x0.x, x0.y, x1.x, x1.y};
                oacc[mt] = mfma_bf16(av, ph, oacc[mt]);
                oacc[mt] = mfma_bf16(av, pl, oacc[mt]);
            }
        } else {
            u32x4 pv[4];
            if constexpr (SRC == SRC_E4M3) {
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4) {
                    float q8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int row = (e < 4) ? 4 * g + e : 16 + 4 * g + (e - 4);
                        q8[e] = p[e >> 2][e & 3] * L.fac[row][b4];
                    }
                    pv[b4] = u32x4{pack_f16_rne(q8[0], q8[1]), pack_f16_rne(q8[2], q8[3]),
                                   pack_f16_rne(q8[4], q8[5]), pack_f16_rne(q8[6], q8[7])};
                }
            } else {
                pv[0] = u32x4{pack_f16_rne(p[0][0], p[0][1]), pack_f16_rne(p[0][2], p[0][3]),
                              pack_f16_rne(p[1][0], p[1][1]), pack_f16_rne(p[1][2], p[1][3])};
            }
#pragma unroll
            for (int mt = 0; mt < kDv / 16; ++mt) {
                const uint16_t* va = L.tile + vt_off(16 * mt + j);
                const u32x2 x0 = *reinterpret_cast<const u32x2*>(va + 4 * g);
                const u32x2 x1 = *reinterpret_cast<const u32x2*>(va + 16 + 4 * g);
                const u32x4 av = u32x4{x0.x, x0.y, x1.x, x1.y};
                oacc[mt] = mfma_f16(av, pv[(SRC == SRC_E4M3) ? (mt >> 3) : 0], oacc[mt]);
            }
        }
    }

    // ---- partial: normalised output and logsumexp (natural log) of the split
    if (!mw) return;
    const int64_t prow = ((int64_t)b * S + split) * a.H + head;
    const float inv_l = (l > 0.0f) ? 1.0f / l : 0.0f;
#pragma unroll
    for (int mt = 0; mt < kDv / 16; ++mt) {
        float f = inv_l;
        if constexpr (SRC == SRC_E4M3) f *= u2f(L.smax_bits[mt >> 3]);
        *reinterpret_cast<float4*>(o_part + prow * kDv + 16 * mt + 4 * g) =
            make_float4(oacc[mt][0] * f, oacc[mt][1] * f, oacc[mt][2] * f, oacc[mt][3] * f);
    }
    if (g == 0)
        lse_part[prow] = (l > 0.0f) ? (m + __builtin_amdgcn_logf(l)) * 0.6931471805599453f : -__builtin_inff();
}

template <int SRC_MAIN, int DQK, int NHT>
__global__ __launch_bounds__(256) void k_decode_mfma(DecodeArgs a, int S_main, int S_win, int rps,
                                                          float* o_part, float* lse_part) {
    __shared__ Lds<DQK> L;
    const int b = blockIdx.y;
    const int split = blockIdx.x;
    const int S = S_main + S_win;
    if (split < S_main) {
        const int64_t first = (int64_t)split * rps;
        const int n = (int)((a.k - first < rps) ? a.k - first : rps);
        decode_split<SRC_MAIN, DQK, NHT>(a, L, b, split, S, false, first, n, o_part, lse_part);
    } else {
        const int64_t first = (int64_t)(split - S_main) * rps;
        const int wl = (int)clamp_visible(a.win_len[b], a.W);
        int n = (int)(wl - first);
        n = n < 0 ? 0 : (n > rps ? rps : n);
        decode_split<SRC_BF16, DQK, NHT>(a, L, b, split, S, true, first, n, o_part, lse_part);
    }
}

// Combine the splits of one (b, h) by their logsumexp; thread t owns channels 4t .. 4t+3.
__global__ __launch_bounds__(kMergeThreads) void k_merge(int S, int H, const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part, float* __restrict__ out,
                                                         float* __restrict__ lse) {
    const int h = blockIdx.x, b = blockIdx.y;
    const int t = threadIdx.x;
    const float* lp = lse_part + (int64_t)b * S * H + h;
    float m = -__builtin_inff();
    for (int s = 0; s < S; ++s) m = fmaxf(m, lp[(int64_t)s * H]);
    float4* o = reinterpret_cast<float4*>(out + ((int64_t)b * H + h) * kDv) + t;
    if (m == -__builtin_inff()) {
        *o = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t == 0) lse[(int64_t)b * H + h] = -__builtin_inff();
        return;
    }
    const float4* op = reinterpret_cast<const float4*>(o_part + ((int64_t)b * S * H + h) * kDv) + t;
    const int64_t step = (int64_t)H * (kDv / 4);
    float tot = 0.0f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int s = 0; s < S; ++s) {
        const float wv = __expf(lp[(int64_t)s * H] - m);
        const float4 v = op[s * step];
        tot += wv;
        acc.x += wv * v.x;
        acc.y += wv * v.y;
        acc.z += wv * v.z;
        acc.w += wv * v.w;
    }
    const float inv = 1.0f / tot;
    *o = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (t == 0) lse[(int64_t)b * H + h] = m + __logf(tot);
}

// ------------------------------------------------------------------------
// Generic path.
__device__ __forceinline__ float e2m1_val(uint32_t n) {
    const uint32_t e = (n >> 1) & 3u, m = n & 1u;
    const float mag = e ? __builtin_ldexpf(1.0f + 0.5f * (float)m, (int)e - 1) : 0.5f * (float)m;
    return (n & 8u) ? -mag : mag;
}

__device__ __forceinline__ float row_elem(int fmt, int dim, const uint8_t* row, int c) {
    switch (fmt) {
    case MLA_FMT_F32: return reinterpret_cast<const float*>(row)[c];
    case MLA_FMT_BF16: return u2f((uint32_t)reinterpret_cast<const uint16_t*>(row)[c] << 16);
    case MLA_FMT_E4M3_S128:
        if (c < dim) return e4m3_to_f32(row[c]) * reinterpret_cast<const float*>(row + dim)[c / 128];
        return u2f((uint32_t)reinterpret_cast<const uint16_t*>(row + dim + 4 * (dim / 128))[c - dim] << 16);
    default: {
        const uint32_t byte = row[c / 2];
        return e2m1_val((c & 1) ? (byte >> 4) : (byte & 15u)) * e4m3_to_f32(row[dim / 2 + c / 16]);
    }
    }
}

__global__ __launch_bounds__(kGenericThreads) void k_decode_generic(DecodeArgs a) {
    __shared__ float zs[kGenericMaxRows];
    __shared__ float qs[1024];
    __shared__ float red[kGenericThreads / 64];
    const int h = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int D = a.dim + a.rope;
    const int n = a.k + (a.win ? a.W : 0);
    for (int c = t; c < D; c += kGenericThreads)
        qs[c] = (a.fmt == MLA_FMT_F32)
                    ? reinterpret_cast<const float*>(a.q)[((int64_t)b * a.H + h) * D + c]
                    : u2f((uint32_t)reinterpret_cast<const uint16_t*>(a.q)[((int64_t)b * a.H + h) * D + c] << 16);
    __syncthreads();
    auto src = [&](int u, bool* win) -> const uint8_t* {
        *win = u >= a.k;
        if (!*win) {
            const int32_t s = a.idx[(int64_t)b * a.k + u];
            if (s < 0 || s >= a.capacity) return nullptr;
            return a.cache + b * a.stride + (int64_t)s * a.row_bytes;
        }
        const int slot = u - a.k;
        if (slot >= clamp_visible(a.win_len[b], a.W)) return nullptr;
        return reinterpret_cast<const uint8_t*>(a.win + ((int64_t)b * a.W + slot) * D);
    };
    float mx = -__builtin_inff();
    for (int u = t; u < n; u += kGenericThreads) {
        bool win;
        const uint8_t* r = src(u, &win);
        float z = -__builtin_inff();
        if (r) {
            float d = 0.0f;
            for (int c = 0; c < D; ++c)
                d += qs[c] * (win ? u2f((uint32_t)reinterpret_cast<const uint16_t*>(r)[c] << 16)
                                  : row_elem(a.fmt, a.dim, r, c));
            z = d * a.scale;
        }
        zs[u] = z;
        mx = fmaxf(mx, z);
    }
    mx = wave_max(mx);
    if ((t & 63) == 0) red[t >> 6] = mx;
    __syncthreads();
    mx = red[0];
    for (int i = 1; i < kGenericThreads / 64; ++i) mx = fmaxf(mx, red[i]);
    __syncthreads();
    float* o = a.out + ((int64_t)b * a.H + h) * a.d_v;
    if (mx == -__builtin_inff()) {
        for (int c = t; c < a.d_v; c += kGenericThreads) o[c] = 0.0f;
        if (t == 0) a.lse[(int64_t)b * a.H + h] = -__builtin_inff();
        return;
    }
    float sum = 0.0f;
    for (int u = t; u < n; u += kGenericThreads) {
        const float p = __expf(zs[u] - mx);
        zs[u] = p;
        sum += p;
    }
    sum = wave_sum(sum);
    if ((t & 63) == 0) red[t >> 6] = sum;
    __syncthreads();
    sum = 0.0f;
    for (int i = 0; i < kGenericThreads / 64; ++i) sum += red[i];
    for (int c = t; c < a.d_v; c += kGenericThreads) {
        float acc = 0.0f;
        for (int u = 0; u < n; ++u) {
            const float p = zs[u];
            if (p == 0.0f) continue;
            bool win;
            const uint8_t* r = src(u, &win);
            acc += p * (win ? u2f((uint32_t)reinterpret_cast<const uint16_t*>(r)[c] << 16)
                            : row_elem(a.fmt, a.dim, r, c));
        }
        o[c] = acc / sum;
    }
    if (t == 0) a.lse[(int64_t)b * a.H + h] = mx + __logf(sum);
}

bool mfma_shape(int fmt, int dim, int rope, int d_v, int H) {
    if (d_v != kDv || (H != 16 && H != 32 && H != 64 && H != 128)) return false;
    if (fmt == MLA_FMT_E4M3_S128) return dim == 512 && rope == 64;
    if (fmt == MLA_FMT_E2M1_S16) return dim == 512 && rope == 0;
    if (fmt == MLA_FMT_BF16) return dim == 512 && (rope == 64 || rope == 0);
    return false;
}

}  // namespace

bool decode_supported(int fmt, int dim, int rope, int d_v, int H) {
    if (mfma_shape(fmt, dim, rope, d_v, H)) return true;
    return dim + rope <= 1024 && d_v <= dim + rope && d_v > 0;
}

static void decode_geometry(int H, int k, int W, int* S_main, int* S_win, int* rps) {
    *rps = rows_per_split(H, k);
    *S_main = (k + *rps - 1) / *rps;
    *S_win = (W + *rps - 1) / *rps;
}

size_t decode_workspace_bytes(int fmt, int dim, int rope, int d_v, int B, int H, int k, int W) {
    if (!mfma_shape(fmt, dim, rope, d_v, H)) return 0;
    int S_main, S_win, rps;
    decode_geometry(H, k, W, &S_main, &S_win, &rps);
    const size_t S = (size_t)(S_main + S_win);
    const size_t o = (size_t)B * S * H * kDv * sizeof(float);
    const size_t l = (size_t)B * S * H * sizeof(float);
    return ((o + 255) & ~(size_t)255) + ((l + 255) & ~(size_t)255);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    if (!mfma_shape(a.fmt, a.dim, a.rope, a.d_v, a.H)) {
        hipLaunchKernelGGL(k_decode_generic, dim3(a.H, a.B), dim3(kGenericThreads), 0, stream, a);
        return hipGetLastError();
    }
    int S_main, S_win, rps;
    decode_geometry(a.H, a.k, a.win ? a.W : 0, &S_main, &S_win, &rps);
    const int S = S_main + S_win;
    const size_t o_bytes = (((size_t)a.B * S * a.H * kDv * sizeof(float)) + 255) & ~(size_t)255;
    float* o_part = reinterpret_cast<float*>(a.workspace);
    float* lse_part = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + o_bytes);
    if (S > 0) {
        const int NHT = a.H >= 64 ? 4 : a.H / 16;
        const dim3 grid(S, a.B, a.H / (16 * NHT));
#define MLA_DEC_CASE(SRC, DQK, N)                                                                      \
    if (NHT == N) {                                                                                    \
        hipLaunchKernelGGL((k_decode_mfma<SRC, DQK, N>), grid, dim3(256), 0, stream, a, S_main,     \
                           S - S_main, rps, o_part, lse_part);                                         \
    }
#define MLA_DEC_ALL_N(SRC, DQK) \
    MLA_DEC_CASE(SRC, DQK, 1) MLA_DEC_CASE(SRC, DQK, 2) MLA_DEC_CASE(SRC, DQK, 4)
        if (a.fmt == MLA_FMT_E4M3_S128) { MLA_DEC_ALL_N(SRC_E4M3, 576) }
        else if (a.fmt == MLA_FMT_E2M1_S16) { MLA_DEC_ALL_N(SRC_FP4, 512) }
        else if (a.rope == 64) { MLA_DEC_ALL_N(SRC_BF16, 576) }
        else { MLA_DEC_ALL_N(SRC_BF16, 512) }
#undef MLA_DEC_ALL_N
#undef MLA_DEC_CASE
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_merge, dim3(a.H, a.B), dim3(kMergeThreads), 0, stream, S, a.H,
                       o_part, lse_part, a.out, a.lse);
    return hipGetLastError();
}

}  // namespace mla
