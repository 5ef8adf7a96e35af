// common.hpp -- device helpers shared by the gfx950 kernels: vector types,
// E4M3 / E2M1 / bf16 codecs, MFMA operand packing, wave reductions.
//
// Format definitions ([P1] "DeepSeek's Attention and KV Cache - From MLA to
// CSA2", "A Precision Primer"): E4M3 "fn" (bias 7, no infinities, one NaN
// pattern, max 448) and E2M1 (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "mla.h"

namespace mla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;

constexpr int kWave = 64;

// ---------------------------------------------------------------- bit casts
__device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// ---------------------------------------------------------------- encoders
// bf16 by round-to-nearest-even of the fp32 bit pattern (NaN -> quiet NaN).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
    uint32_t u = f2u(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E4M3 code of x: round-to-nearest-even on the E4M3 grid, saturating to +-448.
// Sign kept (so -0 -> 0x80).  Works on the fp32 bit pattern.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
    const uint32_t u = f2u(x);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t mag;
    if (a > 0x7F800000u) return 0x7Fu;                      // NaN
    if (a >= 0x43E00000u) {                                 // >= 448
        mag = 0x7Eu;
    } else if (a < 0x3C800000u) {                           // < 2^-6: subnormal step 2^-9
        mag = (uint32_t)__builtin_rintf(u2f(a) * 512.0f);    // exact scaling, RNE to 0..8
    } else {
        int e = (int)(a >> 23) - 127;                       // -6 .. 8
        uint32_t m = a & 0x7FFFFFu;
        uint32_t q = m >> 20;                               // top 3 mantissa bits
        uint32_t rem = m & 0xFFFFFu;
        if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ++q;
        if (q == 8u) { q = 0u; ++e; }
        mag = ((uint32_t)(e + 7) << 3) | q;                 // a < 448 keeps mag <= 0x7E
    }
    return sign | mag;
}

// E2M1 nibble of y: nearest rung, ties to the even mantissa, saturating to +-6.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
    const uint32_t u = f2u(y);
    const uint32_t sign = (u >> 28) & 0x8u;
    const uint32_t a = u & 0x7FFFFFFFu;
    uint32_t mag;
    if (a > 0x7F800000u) return 0x7u;
    if (a >= 0x40C00000u) {                                 // >= 6
        mag = 7u;
    } else if (a < 0x3F800000u) {                           // < 1: step 0.5
        mag = (uint32_t)__builtin_rintf(u2f(a) * 2.0f);      // 0, 1, 2 (2 == 1.0)
    } else {
        int e = (int)(a >> 23) - 127;                       // 0, 1, 2
        uint32_t m = a & 0x7FFFFFu;
        uint32_t q = m >> 22;                               // 1 mantissa bit
        uint32_t rem = m & 0x3FFFFFu;
        if (rem > 0x200000u || (rem == 0x200000u && (q & 1u))) ++q;
        if (q == 2u) { q = 0u; ++e; }
        mag = ((uint32_t)(e + 1) << 1) | q;
        if (mag > 7u) mag = 7u;
    }
    return sign | mag;
}

// Exact value of an E4M3 scale byte as fp32 (scales are never NaN here).
// MXFP4 (OCP microscaling): the E8M0 code of a block whose largest magnitude
// has the fp32 bit pattern `amax_bits` (sign clear): floor(log2 amax) - 2 + 127
// (E2M1's largest value is 1.5 x 2^2), clamped to 0 .. 254, 0 for zeros and
// subnormals; the scale it encodes is 2^(code - 127).
__device__ __forceinline__ uint32_t mx_code(uint32_t amax_bits) {
    const uint32_t e = amax_bits >> 23;
    return e >= 2u ? min(e - 2u, 254u) : 0u;
}
__device__ __forceinline__ float e8m0_to_f32(uint32_t code) {
    return code ? u2f(code << 23) : u2f(0x00400000u);     // code 0: 2^-127, an fp32 subnormal
}
// The E2M1 code of x in an MXFP4 block of code `code` (x / 2^(code - 127), exact
// scaling, then round-to-nearest-even, saturating); zero for a block of zeros.
__device__ __forceinline__ uint32_t mx_encode(float x, uint32_t amax_bits, uint32_t code) {
    return amax_bits ? e2m1_encode(__builtin_ldexpf(x, 127 - (int)code)) : 0u;
}

// E8M0 code of an MXFP8 block (E4M3 elements, largest exponent 8) from the fp32
// bits of its largest magnitude: floor(log2 amax) - 8 + 127, clamped to 0..254.
__device__ __forceinline__ uint32_t mx8_code(uint32_t amax_bits) {
    const uint32_t e = amax_bits >> 23;
    return e >= 8u ? min(e - 8u, 254u) : 0u;
}
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(code & 0xFFu, false);
    return v.x;
}

// ---------------------------------------------------------------- decoders
// Four E4M3 codes (one dword) -> four exact fp32 values.
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* o) {
    f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    o[0] = lo.x; o[1] = lo.y; o[2] = hi.x; o[3] = hi.y;
}

// Pack the bf16 of two fp32 values whose low 16 bits are zero (exact).
__device__ __forceinline__ uint32_t pack_bf16_trunc(float lo, float hi) {
    return __builtin_amdgcn_perm(f2u(hi), f2u(lo), 0x07060302u);
}

// Four E4M3 codes -> two dwords of bf16 (exact: every E4M3 value is a bf16 value;
// the converter's scale operand only contributes its exponent, here 2^0).
__device__ __forceinline__ u32x2 e4m3x4_to_bf16(uint32_t w) {
    u32x2 r;
    r.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
    r.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
    return r;
}

// Byte `sel` (0..3) of w holds two E2M1 nibbles (low nibble = even channel):
// return their values (exact fp32).
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// A caller-supplied count clamped to [0, limit] (keeps every access in bounds).
__device__ __forceinline__ int64_t clamp_visible(int64_t v, int64_t limit) {
    return v < 0 ? 0 : (v > limit ? limit : v);
}

// Workgroup barrier that orders LDS only: the waves' outstanding global stores
// are not waited for (a plain __syncthreads waits for every vector memory
// operation of the wave, stores included, before the barrier).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Order-preserving map of an fp32 score to uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = f2u(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    return u2f((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48, on the VALU: each
// permlane swap hands every lane the value of its partner row (16 lanes) / half.
__device__ __forceinline__ float xmax4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    x = fmaxf(u2f(a[0]), u2f(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return fmaxf(u2f(b[0]), u2f(b[1]));
}
// Sum over lanes l and l ^ 32.
__device__ __forceinline__ float xsum2(float x) {
    const auto b = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return u2f(b[0]) + u2f(b[1]);
}
__device__ __forceinline__ float xsum4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    x = u2f(a[0]) + u2f(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return u2f(b[0]) + u2f(b[1]);
}

// MFMA wrappers (gfx950, 64-lane wave).  Operand layout, verified on the
// device: A lane l holds row (l % 16), k-slots 8*(l/16) .. +7; B lane l holds
// column (l % 16), the same k-slots; D lane l, element r holds row
// 4*(l/16) + r, column l % 16.
typedef __attribute__((ext_vector_type(16))) float f32x16;
// 32x32x16 bf16: lane l holds A[l % 32][8 (l / 32) + e] and B[8 (l / 32) + e][l % 32];
// register v of the result is D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                                  0);
}

// 32x32x64 MFMA on MX operands, E2M1 on both sides: lane (col, g) holds 32
// E2M1 codes (element 2i in the low nibble of byte i) and the E8M0 scale
// (code in the low byte) that applies to those 32 elements; products and their
// sum are exact in the block and the blocks accumulate in fp32.
typedef __attribute__((ext_vector_type(8))) int i32x8;
__device__ __forceinline__ f32x16 mfma32_fp4(u32x4 a, u32x4 b, f32x16 c, uint32_t sa, uint32_t sb) {
    const i32x8 A = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    const i32x8 B = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, c, 4, 4, 0, (int)sa, 0, (int)sb);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Top-k histogram over the high bits of the score key.
constexpr int kHistBits = 12;
constexpr int kHistBins = 1 << kHistBits;
static_assert(kHistBins == kHistBinsHost, "histogram size");
constexpr int kHistCopies = kHistCopiesHost;
constexpr int kCoarseBins = kCoarseBinsHost;
constexpr int kFinePerCoarse = kHistBins / kCoarseBins;
static_assert(kFinePerCoarse == 64, "one fine bin per lane of a wave within a coarse bin");

// Histogram words of sequence b: coarse copy j at hb + 64 j, fine copy j at
// hb + 64 * kHistCopies + 4096 j.
__device__ __forceinline__ uint32_t* hist_coarse(uint32_t* hb, int j) { return hb + kCoarseBins * j; }
__device__ __forceinline__ uint32_t* hist_fine(uint32_t* hb, int j) {
    return hb + kCoarseBins * kHistCopies + kHistBins * j;
}
// The copy a workgroup adds into: the index of the XCD it runs on (hardware
// register XCC_ID), so that every workgroup adding into one copy shares that
// XCD's L2 and the adds can be L2-local atomics; the end of the kernel writes
// the L2 back before any later kernel reads the copies.
__device__ __forceinline__ int hist_copy_of_block() {
    return (int)(__builtin_amdgcn_s_getreg((20 << 0) | (0 << 6) | (3 << 11)) & (kHistCopies - 1));
}
__device__ __forceinline__ void l2_add(uint32_t* p, uint32_t v) {
    __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Add a workgroup's counts into copy j of sequence b's histogram (L2-local
// atomics, see hist_copy_of_block; zero counts skipped). count(i) gives fine bin i's count; the coarse
// bins are the sums of 64 consecutive fine bins. Called by all threads of a
// workgroup of `nthreads` (a multiple of 64) after its counts are final.
template <typename F>
__device__ __forceinline__ void flush_hist_copy(F count, uint32_t* hb, int j, int nthreads) {
    uint32_t* fine = hist_fine(hb, j);
    uint32_t* coarse = hist_coarse(hb, j);
    // thread t covers fine bins 16 q .. 16 q + 15 for q = t, t + nthreads, ..; the 4
    // lanes of a coarse bin (64 fine bins) are adjacent and meet in a shuffle sum
    for (int q = threadIdx.x; q < kHistBins / 16; q += nthreads) {
        uint32_t part = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t c = count(16 * q + i);
            part += c;
            if (c) l2_add(&fine[16 * q + i], c);
        }
        part += __shfl_xor(part, 1, 64);
        part += __shfl_xor(part, 2, 64);
        if ((q & 3) == 0 && part) l2_add(&coarse[q >> 2], part);
    }
}

// ---------------------------------------------------------------- LDS DMA
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Global memory to LDS without passing through registers: every lane's 16 (4)
// bytes land at LDS address m0 + 16 * lane (m0 + 4 * lane). Issued as inline
// assembly so that the compiler neither waits for them at every barrier nor
// reorders them; the kernels wait for them with vmcnt themselves. The compiler
// reserves M0 and warns about the clobber; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* g, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(m0) : "memory", "m0");
}
// wave-uniform base + per-lane 32-bit byte offset
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4_s(const void* sbase, uint32_t voff, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
                 : "memory", "m0");
}
// Device-scope atomic add of 1 by lane 0 alone, returning the old value into r
// (lane 0) once the operation completes. Issued as inline assembly like the
// loads above, so that it joins their in-order vmcnt count; r must not be read
// before a wait_vmcnt_tie on it has covered the operation.
__device__ __forceinline__ void ticket_issue(uint32_t& r, uint32_t* p) {
    uint64_t save;
    asm volatile(
        "s_mov_b64 %1, exec\n\t"
        "s_mov_b64 exec, 1\n\t"
        "s_nop 1\n\t"
        "global_atomic_add %0, %2, %3, off sc0\n\t"
        "s_mov_b64 exec, %1"
        : "=&v"(r), "=&s"(save)
        : "v"(p), "v"(1u)
        : "memory");
}
// Lane 0's value of a ticket register, read after the wait that covers its
// atomic: volatile statements keep their order, so the read cannot move above
// the wait the way an ordinary use of the register could
__device__ __forceinline__ uint32_t ticket_read(uint32_t r) {
    uint32_t t;
    asm volatile("v_readfirstlane_b32 %0, %1" : "=s"(t) : "v"(r));
    return t;
}
#pragma clang diagnostic pop

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// the same wait as a volatile statement, ordered with the other volatile asm
// (ticket_issue, ticket_read) of a wave
template <int N>
__device__ __forceinline__ void wait_vmcnt_asm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace mla
