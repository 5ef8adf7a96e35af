// decode.hip -- absorbed-MLA sparse decode: shared-KV MQA over the selected
// latent entries plus the window, online softmax, logsumexp output.
//
// For each (b, h), over U = {selected rows} + {window slots}:
//   z_u = scale * q[b,h,:] . K_u,  lse = logsumexp z,  out = sum_u e^(z_u - lse) K_u[:d_v]
// ([P1] "DeepSeek's Attention and KV Cache - From MLA to CSA2", "DeepSeek-V2",
// "Why RoPE breaks the trick" and "Check it in numpy"; [P2] "From MLA to DSA
// to HCA/CSA", Part 2 "What replaced MLA"; each selected latent is read once
// for all heads, [P1] "DeepSeek-V3.2", "The lightning indexer").
//
// MFMA path (H = 16 * NHT, d_v = 512, K width 576 = 512 + 64 or 512):
//   grid (splits, B, head groups); a split is `rps` consecutive entries of
//   idx[b] (or of the window ring); workgroup = NHT <= 4 waves (one wave per
//   SIMD: a wave keeps q and the fp32 output tile in registers), wave w owns
//   heads 16 * (NHT * blockIdx.z + w) .. +15.
//   Per 32-row chunk the workgroup gathers the rows once into LDS, dequantised
//   exactly: K row-major in bf16 (E4M3 codes unscaled; E2M1 x scale), V
//   channel-major in fp16 (E4M3 codes / E2M1 x scale, both exact in fp16) or
//   bf16 (bf16 rows).  Each wave computes S^T = K q^T on bf16 MFMA (E4M3: one
//   accumulator per 128-channel block, multiplied by the row's fp32 scale),
//   runs the online softmax in registers and accumulates O^T = V^T P^T on
//   MFMA: fp16 P (E4M3 rows: P times the row scale over the split's largest
//   scale of that block, so P <= 1), or bf16 P split into a high and a low
//   part when V is bf16.  The split's normalised output and its logsumexp are
//   written as a partial; k_merge combines the partials by logsumexp.
// Generic path (any other shape): one workgroup per (b, h), fp32 on the vector
// ALUs, writes the final output directly.
#include <cstdlib>

#include "common.hpp"
#include "launch.hpp"

namespace mla {

namespace {

constexpr int kChunk = 32;
constexpr int kVt = 36;                  // halves per V^T channel row (32 rows + pad)
constexpr int kDv = 512;
constexpr int kMergeThreads = 256;
constexpr int kGenericThreads = 256;
constexpr int kGenericMaxRows = 8192;

enum SrcKind { SRC_E4M3 = 0, SRC_FP4 = 1, SRC_BF16 = 2 };

// Entries per split: fewer splits mean fewer fp32 partials to write and merge,
// more splits mean more workgroups in flight.  MLA_DECODE_RPS (a multiple of
// 32) overrides the default for tuning; the workspace query reads it too.
int rows_per_split(int H, int k) {
    (void)k;
    if (const char* e = getenv("MLA_DECODE_RPS")) {
        const int v = atoi(e);
        if (v >= 32 && v % 32 == 0) return v;
    }
    return H >= 128 ? 256 : 128;
}

template <int DQK>
struct Lds {
    static constexpr int kKs = DQK + 8;                 // bf16 per K / q row (padded)
    uint16_t qs[64 * kKs];                              // q of the workgroup's (up to) 64 heads
    uint16_t ks[kChunk * kKs];
    uint16_t vt[kDv * kVt];
    float rscale[kChunk][4];
    int32_t valid[kChunk];
    uint32_t sref_bits[4];
};

// Raw bytes of one gather item (32 channels of one row) held in registers
// between its global load and its dequantising store into LDS.
struct Slot {
    u32x4 v[4];
    uint32_t x;           // E4M3: the row's fp32 scale word; E2M1: the two scale bytes
    int ok;
};

// Issue the global loads of segment `sg` (channels 32*sg .. +31) of a row.
template <int SRC, int DQK>
__device__ __forceinline__ void load_segment(Slot& sl, const uint8_t* __restrict__ row, int sg) {
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

// Dequantise a loaded segment into LDS row r: K row-major in bf16 and, for the
// value channels, V^T channel-major (fp16 for E4M3 / E2M1, bf16 for bf16 rows).
template <int SRC, int DQK>
__device__ __forceinline__ void store_segment(Lds<DQK>& L, const Slot& sl, int r, int sg) {
    uint16_t* kdst = L.ks + r * Lds<DQK>::kKs + sg * 32;
    const bool in_v = sg * 32 < kDv;
    if constexpr (SRC == SRC_BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) reinterpret_cast<u32x4*>(kdst)[i] = sl.v[i];
        if (in_v) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t w = sl.v[i][e];
                    L.vt[(sg * 32 + 8 * i + 2 * e) * kVt + r] = (uint16_t)(w & 0xFFFFu);
                    L.vt[(sg * 32 + 8 * i + 2 * e + 1) * kVt + r] = (uint16_t)(w >> 16);
                }
        }
    } else if constexpr (SRC == SRC_E4M3) {
        if (sg < 16) {
            const uint32_t w[8] = {sl.v[0].x, sl.v[0].y, sl.v[0].z, sl.v[0].w,
                                   sl.v[1].x, sl.v[1].y, sl.v[1].z, sl.v[1].w};
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                float f[4];
                e4m3x4_to_f32(w[i], f);
                reinterpret_cast<uint32_t*>(kdst)[2 * i] = pack_bf16_trunc(f[0], f[1]);
                reinterpret_cast<uint32_t*>(kdst)[2 * i + 1] = pack_bf16_trunc(f[2], f[3]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    L.vt[(sg * 32 + 4 * i + e) * kVt + r] = __builtin_bit_cast(uint16_t, (_Float16)f[e]);
            }
            if ((sg & 3) == 0) L.rscale[r][sg >> 2] = u2f(sl.x);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) reinterpret_cast<u32x4*>(kdst)[i] = sl.v[i];
        }
    } else {
        const float s0 = e4m3_to_f32(sl.x & 0xFFu), s1 = e4m3_to_f32((sl.x >> 8) & 0xFFu);
        const uint32_t w[4] = {sl.v[0].x, sl.v[0].y, sl.v[0].z, sl.v[0].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = (i < 2) ? s0 : s1;
            f32x2 v[4] = {e2m1x2_to_f32<0>(w[i]), e2m1x2_to_f32<1>(w[i]), e2m1x2_to_f32<2>(w[i]),
                          e2m1x2_to_f32<3>(w[i])};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = v[e].x * s, bb = v[e].y * s;
                reinterpret_cast<uint32_t*>(kdst)[4 * i + e] = pack_bf16_trunc(a, bb);
                L.vt[(sg * 32 + 8 * i + 2 * e) * kVt + r] = __builtin_bit_cast(uint16_t, (_Float16)a);
                L.vt[(sg * 32 + 8 * i + 2 * e + 1) * kVt + r] = __builtin_bit_cast(uint16_t, (_Float16)bb);
            }
        }
    }
}

template <int DQK>
__device__ __forceinline__ void zero_segment(Lds<DQK>& L, int r, int sg) {
    uint16_t* kdst = L.ks + r * Lds<DQK>::kKs + sg * 32;
#pragma unroll
    for (int i = 0; i < 4; ++i) reinterpret_cast<u32x4*>(kdst)[i] = u32x4{0u, 0u, 0u, 0u};
    if (sg * 32 < kDv)
#pragma unroll
        for (int e = 0; e < 32; ++e) L.vt[(sg * 32 + e) * kVt + r] = 0;
    if (sg < 4) L.rscale[r][sg] = 0.0f;      // invalid rows carry zero scales (never NaN)
}

__device__ __forceinline__ uint32_t pack_f16_rne(float a, float b) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
}

// Process one split with source kind SRC.  Returns after writing the partial.
template <int SRC, int DQK, int NHT>
__device__ __forceinline__ void decode_split(const DecodeArgs& a, Lds<DQK>& L, int b, int split, int S,
                                             bool is_win, int64_t first, int n_rows, float* o_part,
                                             float* lse_part) {
    constexpr int NT = DQK / 32;          // k-steps of QK
    constexpr int NSEG = DQK / 32;        // 32-channel segments of a row
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6;
    const int j = lane & 15, g = lane >> 4;
    const int head = 16 * (NHT * (int)blockIdx.z + w) + j;
    constexpr float kLog2e = 1.4426950408889634f;
    const float zscale = a.scale * kLog2e;

    // source row of split entry u (nullptr if invalid)
    auto row_ptr = [&](int u) -> const uint8_t* {
        if (u >= n_rows) return nullptr;
        if (is_win) return reinterpret_cast<const uint8_t*>(a.win + ((int64_t)b * a.W + first + u) * DQK);
        const int32_t s = a.idx[(int64_t)b * a.k + first + u];
        if (s < 0 || s >= a.capacity) return nullptr;
        return a.cache + b * a.stride + (int64_t)s * a.row_bytes;
    };

    // gather items of a chunk: (segment, row), segment-major; each thread owns NSLOT of them
    constexpr int NTH = NHT * 64;
    constexpr int NITEMS = kChunk * NSEG;
    constexpr int NSLOT = (NITEMS + NTH - 1) / NTH;
    auto load_chunk = [&](int c0, Slot* sl) {
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            const int item = tid + i * NTH;
            sl[i].ok = 0;
            if (item < NITEMS) {
                const uint8_t* rp = row_ptr(c0 + item % kChunk);
                if (rp) {
                    sl[i].ok = 1;
                    load_segment<SRC, DQK>(sl[i], rp, item / kChunk);
                }
            }
        }
    };
    auto store_chunk = [&](const Slot* sl) {
#pragma unroll
        for (int i = 0; i < NSLOT; ++i) {
            const int item = tid + i * NTH;
            if (item < NITEMS) {
                const int sg = item / kChunk, r = item % kChunk;
                if (sl[i].ok) store_segment<SRC, DQK>(L, sl[i], r, sg);
                else zero_segment<DQK>(L, r, sg);
                if (sg == 0) L.valid[r] = sl[i].ok;
            }
        }
    };
    Slot sl[NSLOT];
    if (n_rows > 0) load_chunk(0, sl);

    // q of the workgroup's heads into LDS (16-byte pieces); lane (j, g) later reads
    // k-slots (g, e) of k-step t = channel t*32 + g*8 + e of head j of its tile
    {
        const int head0 = 16 * NHT * (int)blockIdx.z;
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.H + head0) * DQK;
        for (int i = tid; i < 16 * NHT * (DQK / 8); i += NHT * 64) {
            const int hh = i / (DQK / 8), c8 = i % (DQK / 8);
            *reinterpret_cast<u32x4*>(L.qs + hh * Lds<DQK>::kKs + c8 * 8) =
                *reinterpret_cast<const u32x4*>(qp + (int64_t)hh * DQK + c8 * 8);
        }
    }
    const uint16_t* qrow = L.qs + (16 * w + j) * Lds<DQK>::kKs + g * 8;

    float inv_sref[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (SRC == SRC_E4M3) {
        if (tid < 4) L.sref_bits[tid] = 0u;
        __syncthreads();
        for (int u = tid; u < n_rows; u += NHT * 64) {
            const uint8_t* rp = row_ptr(u);
            if (rp) {
                const float4 sc = *reinterpret_cast<const float4*>(rp + 512);
                atomicMax(&L.sref_bits[0], f2u(sc.x));
                atomicMax(&L.sref_bits[1], f2u(sc.y));
                atomicMax(&L.sref_bits[2], f2u(sc.z));
                atomicMax(&L.sref_bits[3], f2u(sc.w));
            }
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = u2f(L.sref_bits[i]);
            inv_sref[i] = (s > 0.0f) ? 1.0f / s : 1.0f;
        }
    }

    f32x4 oacc[kDv / 16];
#pragma unroll
    for (int i = 0; i < kDv / 16; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -__builtin_inff(), l_run = 0.0f;

    for (int c0 = 0; c0 < n_rows; c0 += kChunk) {
        store_chunk(sl);
        __syncthreads();
        if (c0 + kChunk < n_rows) load_chunk(c0 + kChunk, sl);   // in flight during the MFMAs

        // ---- S^T = K q^T for the chunk's two 16-row tiles
        float z[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const uint16_t* ka = L.ks + (16 * rt + j) * Lds<DQK>::kKs + g * 8;
            f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (SRC == SRC_E4M3) {
#pragma unroll
                for (int b4 = 0; b4 < 4; ++b4) {
                    f32x4 t4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int t = 4 * b4; t < 4 * b4 + 4; ++t)
                        t4 = mfma_bf16(*reinterpret_cast<const u32x4*>(ka + t * 32),
                                       *reinterpret_cast<const u32x4*>(qrow + t * 32), t4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) s[r] += t4[r] * L.rscale[16 * rt + 4 * g + r][b4];
                }
#pragma unroll
                for (int t = 16; t < NT; ++t)
                    s = mfma_bf16(*reinterpret_cast<const u32x4*>(ka + t * 32),
                                  *reinterpret_cast<const u32x4*>(qrow + t * 32), s);
            } else {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    s = mfma_bf16(*reinterpret_cast<const u32x4*>(ka + t * 32),
                                  *reinterpret_cast<const u32x4*>(qrow + t * 32), s);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                z[rt][r] = L.valid[16 * rt + 4 * g + r] ? s[r] * zscale : -__builtin_inff();
        }

        // ---- online softmax (base 2), per head j; lanes j, j+16, j+32, j+48 share a head.
        // The reference m_ref moves only when a chunk's max exceeds it by more than 8
        // (p <= 2^8 keeps fp16 P finite), so the output tile is rarely rescaled.
        float zmax = -__builtin_inff();
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) zmax = fmaxf(zmax, z[rt][r]);
        zmax = fmaxf(zmax, __shfl_xor(zmax, 16, 64));
        zmax = fmaxf(zmax, __shfl_xor(zmax, 32, 64));
        const bool move = zmax > m_run + 8.0f;
        if (__ballot(move)) {
            const float m_new = move ? zmax : m_run;
            const float alpha = (m_run == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < kDv / 16; ++i) oacc[i] *= alpha;
            m_run = m_new;
        }
        float p[2][4];
        float psum = 0.0f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                p[rt][r] = (z[rt][r] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(z[rt][r] - m_run);
                psum += p[rt][r];
            }
        psum += __shfl_xor(psum, 16, 64);
        psum += __shfl_xor(psum, 32, 64);
        l_run += psum;

        // ---- O^T += V^T P^T.  k-slot (g, e): e < 4 -> row 4g+e, e >= 4 -> row 16+4g+e-4
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
                const uint16_t* va = L.vt + (16 * mt + j) * kVt;
                const u32x2 v0 = *reinterpret_cast<const u32x2*>(va + 4 * g);
                const u32x2 v1 = *reinterpret_cast<const u32x2*>(va + 16 + 4 * g);
                const u32x4 av = u32x4{v0.x, v0.y, v1.x, v1.y};
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
                        q8[e] = p[e >> 2][e & 3] * (L.rscale[row][b4] * inv_sref[b4]);
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
                const uint16_t* va = L.vt + (16 * mt + j) * kVt;
                const u32x2 v0 = *reinterpret_cast<const u32x2*>(va + 4 * g);
                const u32x2 v1 = *reinterpret_cast<const u32x2*>(va + 16 + 4 * g);
                const u32x4 av = u32x4{v0.x, v0.y, v1.x, v1.y};
                oacc[mt] = mfma_f16(av, pv[(SRC == SRC_E4M3) ? (mt >> 3) : 0], oacc[mt]);
            }
        }
        __syncthreads();
    }

    // ---- partial: normalised output and logsumexp (natural log) of the split
    const int64_t prow = ((int64_t)b * S + split) * a.H + head;
    const float inv_l = (l_run > 0.0f) ? 1.0f / l_run : 0.0f;
#pragma unroll
    for (int mt = 0; mt < kDv / 16; ++mt) {
        float f = inv_l;
        if constexpr (SRC == SRC_E4M3) f *= u2f(L.sref_bits[mt >> 3]);
        float4 v = make_float4(oacc[mt][0] * f, oacc[mt][1] * f, oacc[mt][2] * f, oacc[mt][3] * f);
        *reinterpret_cast<float4*>(o_part + prow * kDv + 16 * mt + 4 * g) = v;
    }
    if (g == 0)
        lse_part[prow] = (l_run > 0.0f) ? (m_run + __builtin_amdgcn_logf(l_run)) * 0.6931471805599453f
                                        : -__builtin_inff();
}

template <int SRC_MAIN, int DQK, int NHT>
__global__ __launch_bounds__(NHT * 64) void k_decode_mfma(DecodeArgs a, int S_main, int S_win, int rps,
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

__global__ __launch_bounds__(kMergeThreads) void k_merge(int S, int H, const float* __restrict__ o_part,
                                                         const float* __restrict__ lse_part, float* __restrict__ out,
                                                         float* __restrict__ lse) {
    extern __shared__ float wts[];
    const int h = blockIdx.x, b = blockIdx.y;
    float m = -__builtin_inff();
    for (int s = 0; s < S; ++s) m = fmaxf(m, lse_part[((int64_t)b * S + s) * H + h]);
    float* o = out + ((int64_t)b * H + h) * kDv;
    if (m == -__builtin_inff()) {
        for (int c = threadIdx.x; c < kDv; c += kMergeThreads) o[c] = 0.0f;
        if (threadIdx.x == 0) lse[(int64_t)b * H + h] = -__builtin_inff();
        return;
    }
    float tot = 0.0f;
    for (int s = 0; s < S; ++s) {
        const float wv = __expf(lse_part[((int64_t)b * S + s) * H + h] - m);
        if (threadIdx.x == 0) wts[s] = wv;
        tot += wv;
    }
    __syncthreads();
    const float inv = 1.0f / tot;
    for (int c = threadIdx.x; c < kDv; c += kMergeThreads) {
        float acc = 0.0f;
        for (int s = 0; s < S; ++s) acc += wts[s] * o_part[(((int64_t)b * S + s) * H + h) * kDv + c];
        o[c] = acc * inv;
    }
    if (threadIdx.x == 0) lse[(int64_t)b * H + h] = m + __logf(tot);
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
        hipLaunchKernelGGL((k_decode_mfma<SRC, DQK, N>), grid, dim3(N * 64), 0, stream, a, S_main,     \
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
    hipLaunchKernelGGL(k_merge, dim3(a.H, a.B), dim3(kMergeThreads), S * sizeof(float), stream, S, a.H,
                       o_part, lse_part, a.out, a.lse);
    return hipGetLastError();
}

}  // namespace mla
