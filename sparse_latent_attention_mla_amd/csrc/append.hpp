// append.hpp -- quantise-append of one new entry, shared by the append kernel
// and the indexer scan that carries the append of its own step.
//
// The entry is quantised after RoPE with block scales only ([P1] "DeepSeek's
// Attention and KV Cache - From MLA to CSA2", "DeepSeek-V4.1", "Four bits for
// the main KV, eight for the window"; 656 / 132-byte V3.2 rows: "DeepSeek-V3.2",
// "What it costs and what it saves"). Quantisation is bit-exact with the row
// format definitions in mla.h: the block maximum, the fp32 divisions and the
// round-to-nearest-even encoders are the only arithmetic.
#pragma once

#include "common.hpp"
#include "launch.hpp"

namespace mla {

constexpr int kStageMain = 2048;           // rows up to these sizes are staged through LDS
constexpr int kStageIdx = 1024;
// LDS one entry needs: block maxima, then the staged main and indexer rows (fp32)
constexpr int kAppendLdsBytes = 64 * 4 + (kStageMain + kStageIdx) * 4;

// Quantise one row of `dim + rope` fp32 values into `dst` (row_bytes bytes) with
// NT threads. `amax_bits` is LDS scratch of at least dim/16 uints.
template <int NT>
__device__ void quant_row(int fmt, int dim, int rope, const float* __restrict__ src, uint8_t* __restrict__ dst,
                          uint32_t* amax_bits) {
    const int t = threadIdx.x;
    if (fmt == MLA_FMT_F32) {
        for (int c = t; c < dim + rope; c += NT) reinterpret_cast<float*>(dst)[c] = src[c];
        return;
    }
    if (fmt == MLA_FMT_BF16) {
        for (int c = t; c < dim + rope; c += NT) reinterpret_cast<uint16_t*>(dst)[c] = (uint16_t)bf16_rne(src[c]);
        return;
    }
    const int blk = (fmt == MLA_FMT_E4M3_S128) ? 128 : ((fmt == MLA_FMT_MXFP4 || fmt == MLA_FMT_MXFP8) ? 32 : 16);
    const int nblk = dim / blk;
    for (int j = t; j < nblk; j += NT) amax_bits[j] = 0u;
    __syncthreads();
    for (int c = t; c < dim; c += NT) atomicMax(&amax_bits[c / blk], f2u(fabsf(src[c])));
    __syncthreads();
    if (fmt == MLA_FMT_E4M3_S128) {
        float* scales = reinterpret_cast<float*>(dst + dim);     // dim is a multiple of 128
        for (int c = t; c < dim; c += NT) {
            const float a = u2f(amax_bits[c / 128]);
            const float s = a / 448.0f;
            dst[c] = (a == 0.0f) ? (uint8_t)0 : (uint8_t)e4m3_encode(src[c] / s);
        }
        for (int j = t; j < nblk; j += NT) scales[j] = u2f(amax_bits[j]) / 448.0f;
        uint16_t* ropep = reinterpret_cast<uint16_t*>(dst + dim + 4 * nblk);
        for (int r = t; r < rope; r += NT) ropep[r] = (uint16_t)bf16_rne(src[dim + r]);
    } else if (fmt == MLA_FMT_MXFP8) {                     // x / X by an exact power of two
        for (int c = t; c < dim; c += NT) {
            const uint32_t ab = amax_bits[c / 32];
            dst[c] = ab == 0u ? (uint8_t)0 : (uint8_t)e4m3_encode(__builtin_ldexpf(src[c], 127 - (int)mx8_code(ab)));
        }
        for (int j = t; j < nblk; j += NT) dst[dim + j] = (uint8_t)mx8_code(amax_bits[j]);
    } else if (fmt == MLA_FMT_MXFP4) {
        for (int p = t; p < dim / 2; p += NT) {
            const int c = 2 * p;
            const uint32_t ab = amax_bits[c / 32], code = mx_code(ab);
            dst[p] = (uint8_t)(mx_encode(src[c], ab, code) | (mx_encode(src[c + 1], ab, code) << 4));
        }
        for (int j = t; j < nblk; j += NT) dst[dim / 2 + j] = (uint8_t)mx_code(amax_bits[j]);
    } else {  // MLA_FMT_E2M1_S16
        for (int p = t; p < dim / 2; p += NT) {
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
        for (int j = t; j < nblk; j += NT) dst[dim / 2 + j] = (uint8_t)e4m3_encode(u2f(amax_bits[j]) / 6.0f);
    }
}

// The same quantisation of 128 channels (one E4M3 block, 8 E2M1 blocks of 16
// or 4 MXFP4 blocks of 32) by one wave, in registers: lane l holds channels 2l
// and 2l + 1 (v0, v1) and writes their codes (E4M3: codes[2l .. 2l + 1]; E2M1
// and MXFP4: the byte codes[l]); the block scale goes to `scales` (E4M3: one
// fp32; E2M1: 8 E4M3 bytes; MXFP4: 4 E8M0 bytes). Block maxima are wave,
// 8-lane or 16-lane maxima of the same fp32 bit patterns quant_row takes, so
// every byte equals quant_row's. Pointers may be global or LDS; E4M3 `scales`
// must be 4-byte aligned.
template <int FMT>
__device__ __forceinline__ void quant128_wave(float v0, float v1, uint8_t* codes, uint8_t* scales) {
    const int l = threadIdx.x & 63;
    uint32_t m = max(f2u(fabsf(v0)), f2u(fabsf(v1)));
    if constexpr (FMT == MLA_FMT_E4M3_S128) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
        const float a = u2f(m);
        const float s = a / 448.0f;
        const uint32_t c0 = (a == 0.0f) ? 0u : e4m3_encode(v0 / s);
        const uint32_t c1 = (a == 0.0f) ? 0u : e4m3_encode(v1 / s);
        reinterpret_cast<uint16_t*>(codes)[l] = (uint16_t)(c0 | (c1 << 8));
        if (l == 0) *reinterpret_cast<float*>(scales) = a / 448.0f;
    } else {
#pragma unroll
        for (int o = 4; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
        const uint32_t sc = e4m3_encode(u2f(m) / 6.0f);
        const float sf = e4m3_to_f32(sc);
        uint32_t lo = 0u, hi = 0u;
        if (sf != 0.0f) {
            lo = e2m1_encode(v0 / sf);
            hi = e2m1_encode(v1 / sf);
        }
        codes[l] = (uint8_t)(lo | (hi << 4));
        if ((l & 7) == 0) scales[l >> 3] = (uint8_t)sc;
    }
}
template <>
__device__ __forceinline__ void quant128_wave<MLA_FMT_MXFP4>(float v0, float v1, uint8_t* codes, uint8_t* scales) {
    const int l = threadIdx.x & 63;
    uint32_t m = max(f2u(fabsf(v0)), f2u(fabsf(v1)));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    const uint32_t code = mx_code(m);
    codes[l] = (uint8_t)(mx_encode(v0, m, code) | (mx_encode(v1, m, code) << 4));
    if ((l & 15) == 0) scales[l >> 4] = (uint8_t)code;
}

// MXFP8 quantisation of the first n (a multiple of 32, at most 128) channels
// by one wave: lane l holds channels 2l and 2l + 1, a block of 32 channels is
// a group of 16 lanes (its maximum by shuffles), codes[2l .. 2l + 1] and
// scales[j] of block j are written; every byte equals quant_row's. `codes`
// must be 2-byte aligned.
__device__ __forceinline__ void quant_mx8_wave(float v0, float v1, int n, uint8_t* codes, uint8_t* scales) {
    const int l = threadIdx.x & 63;
    uint32_t m = max(f2u(fabsf(v0)), f2u(fabsf(v1)));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o, 64));
    const uint32_t code = mx8_code(m);
    const int sh = 127 - (int)code;
    const uint32_t c0 = m == 0u ? 0u : e4m3_encode(__builtin_ldexpf(v0, sh));
    const uint32_t c1 = m == 0u ? 0u : e4m3_encode(__builtin_ldexpf(v1, sh));
    if (2 * l < n) reinterpret_cast<uint16_t*>(codes)[l] = (uint16_t)(c0 | (c1 << 8));
    if ((l & 15) == 0 && 2 * l < n) scales[l >> 4] = (uint8_t)code;
}

// An entry cut into pieces of at most 128 channels that one wave each
// quantises in registers (no LDS, no barrier): for entry e = (b, i), the main
// row's 128-channel blocks, its RoPE part (at most 128 channels, bf16), the
// indexer key (128 channels), and for i == 0 the window entry in slices of 128
// (bf16). Main rows E4M3 or E2M1 with dim a multiple of 128, indexer keys of
// 128 channels; the rows and window entry must be 8-byte aligned.
struct PieceMap {
    int main_blocks, rope, per_entry, win_pieces;
};

__host__ __device__ inline PieceMap piece_map(const AppendArgs& a) {
    PieceMap m;
    m.main_blocks = a.main_cache ? a.main_dim / 128 : 0;
    m.rope = (a.main_cache && a.main_rope > 0) ? 1 : 0;
    m.per_entry = m.main_blocks + m.rope + (a.idx_cache ? 1 : 0);
    m.win_pieces = a.win_ring ? (a.Dw + 127) / 128 : 0;
    return m;
}
__host__ inline int64_t piece_count(const AppendArgs& a) {
    const PieceMap m = piece_map(a);
    return (int64_t)a.B * (a.n_new * m.per_entry + m.win_pieces);
}
__host__ inline bool pieces_supported(const AppendArgs& a) {
    if (a.win_ring && a.win_fmt == MLA_FMT_MXFP8 &&                 // 2-byte aligned entries
        (((a.Dw / 32) & 1) != 0 || reinterpret_cast<uintptr_t>(a.win_ring) % 2 != 0))
        return false;
    if (a.main_cache && !((a.main_fmt == MLA_FMT_E4M3_S128 && a.main_rope <= 128) ||
                          (a.main_fmt == MLA_FMT_E2M1_S16 && a.main_rope == 0) ||
                          (a.main_fmt == MLA_FMT_BF16 && a.main_rope <= 128)))
        return false;
    if (a.main_cache && a.main_dim % 128 != 0) return false;
    if (a.idx_cache && !((a.idx_fmt == MLA_FMT_E4M3_S128 || a.idx_fmt == MLA_FMT_E2M1_S16 ||
                          a.idx_fmt == MLA_FMT_MXFP4 || a.idx_fmt == MLA_FMT_BF16) && a.idx_dim == 128))
        return false;
    // bf16 rows are written two channels (4 bytes) per lane
    if (a.main_cache && a.main_fmt == MLA_FMT_BF16 &&
        (reinterpret_cast<uintptr_t>(a.main_cache) % 4 != 0 || a.main_stride % 4 != 0 || a.main_row_bytes % 4 != 0))
        return false;
    if (a.idx_cache && a.idx_fmt == MLA_FMT_BF16 &&
        (reinterpret_cast<uintptr_t>(a.idx_cache) % 4 != 0 || a.idx_stride % 4 != 0 || a.idx_row_bytes % 4 != 0))
        return false;
    return reinterpret_cast<uintptr_t>(a.new_main) % 8 == 0 && reinterpret_cast<uintptr_t>(a.new_idx) % 8 == 0 &&
           reinterpret_cast<uintptr_t>(a.new_win) % 8 == 0 && (a.main_dim + a.main_rope) % 2 == 0 &&
           a.Dw % 2 == 0;
}

// Piece p of the append, held by one wave between its load and its store.
struct Piece {
    int kind;          // 0 none, 1 main block, 2 rope, 3 indexer key, 4 window slice
    int part, n, b;    // block / slice index, channels, sequence
    int64_t slot;      // row (main, rope, key) or window position
    float v0, v1;      // channels 2l, 2l + 1 of the piece (lane l)
};

__device__ __forceinline__ void piece_load(const AppendArgs& a, int64_t p, Piece& pc) {
    const int l = threadIdx.x & 63;
    const PieceMap m = piece_map(a);
    pc.kind = 0;
    pc.v0 = pc.v1 = 0.0f;
    const int64_t per_b = (int64_t)a.n_new * m.per_entry + m.win_pieces;
    if (p < 0 || p >= (int64_t)a.B * per_b) return;
    const int b = (int)(p / per_b);
    int r = (int)(p - (int64_t)b * per_b);
    pc.b = b;
    const float* src = nullptr;
    if (r < a.n_new * m.per_entry) {
        const int i = r / m.per_entry, q = r - i * m.per_entry;
        const int64_t e = (int64_t)b * a.n_new + i;
        pc.slot = a.slots[e];
        if (q < m.main_blocks) {
            pc.kind = 1; pc.part = q; pc.n = 128;
            src = a.new_main + e * (a.main_dim + a.main_rope) + 128 * q;
        } else if (q < m.main_blocks + m.rope) {
            pc.kind = 2; pc.part = 0; pc.n = a.main_rope;
            src = a.new_main + e * (a.main_dim + a.main_rope) + a.main_dim;
        } else {
            pc.kind = 3; pc.part = 0; pc.n = 128;
            src = a.new_idx + e * 128;
        }
    } else {
        const int q = r - a.n_new * m.per_entry;
        pc.kind = 4; pc.part = q; pc.n = min(128, a.Dw - 128 * q);
        pc.slot = a.win_pos[b];
        src = a.new_win + (int64_t)b * a.Dw + 128 * q;
    }
    if (2 * l < pc.n) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(src + 2 * l);
        pc.v0 = v.x;
        pc.v1 = v.y;
    }
}

__device__ __forceinline__ void piece_store(const AppendArgs& a, const Piece& pc) {
    const int l = threadIdx.x & 63;
    if (pc.kind == 0) return;
    if (pc.kind == 4 && a.win_fmt == MLA_FMT_MXFP8) {      // window slice, MXFP8 (n % 32 == 0)
        if (pc.slot < 0) return;
        uint8_t* ent = reinterpret_cast<uint8_t*>(a.win_ring) + ((int64_t)pc.b * a.W + pc.slot % a.W) * (a.Dw + a.Dw / 32);
        quant_mx8_wave(pc.v0, pc.v1, pc.n, ent + 128 * pc.part, ent + a.Dw + 4 * pc.part);
        return;
    }
    if (pc.kind == 4) {                                    // window slice, bf16
        if (pc.slot < 0) return;
        uint16_t* dst = a.win_ring + ((int64_t)pc.b * a.W + pc.slot % a.W) * a.Dw + 128 * pc.part;
        if (2 * l < pc.n) reinterpret_cast<uint32_t*>(dst)[l] = bf16_rne(pc.v0) | (bf16_rne(pc.v1) << 16);
        return;
    }
    if (pc.slot < 0 || pc.slot >= a.capacity) return;
    if (pc.kind == 3) {                                    // indexer key
        uint8_t* row = a.idx_cache + pc.b * a.idx_stride + pc.slot * a.idx_row_bytes;
        if (a.idx_fmt == MLA_FMT_BF16) {                   // (2 l < 128 for every lane)
            reinterpret_cast<uint32_t*>(row)[l] = bf16_rne(pc.v0) | (bf16_rne(pc.v1) << 16);
            return;
        }
        if (a.idx_fmt == MLA_FMT_E4M3_S128) quant128_wave<MLA_FMT_E4M3_S128>(pc.v0, pc.v1, row, row + 128);
        else if (a.idx_fmt == MLA_FMT_MXFP4) quant128_wave<MLA_FMT_MXFP4>(pc.v0, pc.v1, row, row + 64);
        else quant128_wave<MLA_FMT_E2M1_S16>(pc.v0, pc.v1, row, row + 64);
        return;
    }
    uint8_t* row = a.main_cache + pc.b * a.main_stride + pc.slot * a.main_row_bytes;
    if (a.main_fmt == MLA_FMT_BF16) {                      // bf16 row: block `part`, or the RoPE part
        uint8_t* dst = row + 2 * (pc.kind == 2 ? a.main_dim : 128 * pc.part);
        if (2 * l < pc.n) reinterpret_cast<uint32_t*>(dst)[l] = bf16_rne(pc.v0) | (bf16_rne(pc.v1) << 16);
        return;
    }
    if (pc.kind == 2) {                                    // RoPE part of an E4M3 row, bf16
        uint8_t* rp = row + a.main_dim + 4 * (a.main_dim / 128);
        if (2 * l < pc.n) {
            reinterpret_cast<uint16_t*>(rp)[2 * l] = (uint16_t)bf16_rne(pc.v0);
            reinterpret_cast<uint16_t*>(rp)[2 * l + 1] = (uint16_t)bf16_rne(pc.v1);
        }
        return;
    }
    if (a.main_fmt == MLA_FMT_E4M3_S128)
        quant128_wave<MLA_FMT_E4M3_S128>(pc.v0, pc.v1, row + 128 * pc.part, row + a.main_dim + 4 * pc.part);
    else
        quant128_wave<MLA_FMT_E2M1_S16>(pc.v0, pc.v1, row + 64 * pc.part, row + a.main_dim / 2 + 8 * pc.part);
}

// Entry i of sequence b (a block of NT threads): its quantised main row and
// indexer key at row slots[b, i] and, for i == 0, the bf16 window entry at ring
// slot win_pos[b] mod W. append_load issues every global load of the entry at
// once (slot, new rows, window entry) into registers, so the block pays one
// memory round trip; append_store stages the rows in LDS (`lds`,
// kAppendLdsBytes) for the quantisers and writes the caches. A kernel may run
// other work between the two.
template <int NT>
struct AppendStage {
    float vm[kStageMain / NT], vi[(kStageIdx + NT - 1) / NT], vw[kStageMain / NT];
    int64_t slot;
    int pos;
};

template <int NT>
__device__ __forceinline__ void append_load(const AppendArgs& a, int i, int b, AppendStage<NT>& st) {
    const int t = threadIdx.x;
    const bool rows = (a.main_cache || a.idx_cache) && i < a.n_new;
    const int D = a.main_dim + a.main_rope;
    const int64_t e = (int64_t)b * a.n_new + i;
    const float* gmain = (rows && a.main_cache) ? a.new_main + e * D : nullptr;
    const float* gidx = (rows && a.idx_cache) ? a.new_idx + e * a.idx_dim : nullptr;
    const bool stage = D <= kStageMain && a.idx_dim <= kStageIdx;
    st.slot = rows ? a.slots[e] : -1;
    if (stage) {
#pragma unroll
        for (int j = 0; j < kStageMain / NT; ++j) {
            const int c = t + NT * j;
            st.vm[j] = (gmain && c < D) ? gmain[c] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < (kStageIdx + NT - 1) / NT; ++j) {
            const int c = t + NT * j;
            st.vi[j] = (gidx && c < a.idx_dim) ? gidx[c] : 0.0f;
        }
    }
    const bool win = a.win_ring && i == 0;
    st.pos = win ? a.win_pos[b] : -1;
    if (win && a.Dw <= kStageMain) {
        const float* wsrc = a.new_win + (int64_t)b * a.Dw;
#pragma unroll
        for (int j = 0; j < kStageMain / NT; ++j) {
            const int c = t + NT * j;
            st.vw[j] = (c < a.Dw) ? wsrc[c] : 0.0f;
        }
    }
}

template <int NT>
__device__ void append_store(const AppendArgs& a, int i, int b, const AppendStage<NT>& st, uint8_t* lds) {
    uint32_t* amax_bits = reinterpret_cast<uint32_t*>(lds);       // dim/16 <= 64, dim/128 <= 64
    float* s_main = reinterpret_cast<float*>(lds + 256);
    float* s_idx = s_main + kStageMain;
    const int t = threadIdx.x;
    const bool rows = (a.main_cache || a.idx_cache) && i < a.n_new;
    const int D = a.main_dim + a.main_rope;
    const int64_t e = (int64_t)b * a.n_new + i;
    const float* gmain = (rows && a.main_cache) ? a.new_main + e * D : nullptr;
    const float* gidx = (rows && a.idx_cache) ? a.new_idx + e * a.idx_dim : nullptr;
    const bool stage = D <= kStageMain && a.idx_dim <= kStageIdx;
    const int64_t slot = st.slot;
    if (stage) {
#pragma unroll
        for (int j = 0; j < kStageMain / NT; ++j) s_main[t + NT * j] = st.vm[j];
#pragma unroll
        for (int j = 0; j < (kStageIdx + NT - 1) / NT; ++j)
            if (t + NT * j < kStageIdx) s_idx[t + NT * j] = st.vi[j];
        __syncthreads();
    }
    if (rows && slot >= 0 && slot < a.capacity) {
        if (gmain) {
            quant_row<NT>(a.main_fmt, a.main_dim, a.main_rope, stage ? s_main : gmain,
                          a.main_cache + b * a.main_stride + slot * a.main_row_bytes, amax_bits);
            __syncthreads();
        }
        if (gidx)
            quant_row<NT>(a.idx_fmt, a.idx_dim, 0, stage ? s_idx : gidx,
                          a.idx_cache + b * a.idx_stride + slot * a.idx_row_bytes, amax_bits);
    }
    const bool win = a.win_ring && i == 0;
    if (win && st.pos >= 0 && a.win_fmt == MLA_FMT_MXFP8) {   // (Dw <= kStageMain)
        uint8_t* dst = reinterpret_cast<uint8_t*>(a.win_ring) + ((int64_t)b * a.W + st.pos % a.W) * (a.Dw + a.Dw / 32);
        __syncthreads();                                   // the rows' quantisers are done with the LDS
#pragma unroll
        for (int j = 0; j < kStageMain / NT; ++j)
            if (t + NT * j < a.Dw) s_main[t + NT * j] = st.vw[j];
        __syncthreads();
        quant_row<NT>(MLA_FMT_MXFP8, a.Dw, 0, s_main, dst, amax_bits);
    } else if (win && st.pos >= 0) {
        const float* wsrc = a.new_win + (int64_t)b * a.Dw;
        uint16_t* dst = a.win_ring + ((int64_t)b * a.W + st.pos % a.W) * a.Dw;
        if (a.Dw <= kStageMain) {
#pragma unroll
            for (int j = 0; j < kStageMain / NT; ++j) {
                const int c = t + NT * j;
                if (c < a.Dw) dst[c] = (uint16_t)bf16_rne(st.vw[j]);
            }
        } else {
            for (int c = t; c < a.Dw; c += NT) dst[c] = (uint16_t)bf16_rne(wsrc[c]);
        }
    }
}

}  // namespace mla
