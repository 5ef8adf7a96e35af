/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark.  The HIP library never includes, links or
 * calls it, and it shares no code with the HIP library.
 *
 * Sources (web pages; cited by title and section):
 *  [P1] "DeepSeek's Attention and KV Cache - From MLA to CSA2, From First
 *       Principles" (monishver11.github.io)
 *  [P2] "From MLA to DSA to HCA/CSA: DeepSeek V3.2 and V4 Attention"
 *       (niyunsheng.github.io)
 *  [P3] "DeepSeek-V4.1-Flash and the 890-byte KV cache" (aigenapps.com)
 *  [P4] "From First Principles: DeepSeek-V4.1-Flash Inference" (efekaya.co)
 *
 * Precision: every dot product, softmax and log-sum-exp is accumulated in
 * double; quantisation decisions are taken in fp32 exactly as the formats
 * define them; results are rounded to fp32 once, at the end.
 *
 * Parity pins (what this file is checked against, outside itself) are listed
 * with each function.  Functions without one would say "parity unpinned".
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops use from now on (n >= 1); for timing the oracle on one core. */
void orc_set_threads(int n) {
    if (n >= 1) omp_set_num_threads(n);
}

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Round a non-negative, exactly representable double to the nearest integer,
 * ties to the even integer (IEEE round-to-nearest-even on an integer grid). */
static double rne_int(double v) {
    double f = floor(v);
    double r = v - f;
    if (r > 0.5) return f + 1.0;
    if (r < 0.5) return f;
    return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;
}

/* ------------------------------------------------------------------------- */
/* E4M3 ("fn" variant): [P1] "A Precision Primer", FP8: E4M3 and E5M2 -- no
 * infinities, a single NaN pattern, 18 binades, largest finite 448.
 * Bits s|eeee|mmm, exponent bias 7.  e > 0: 2^(e-7) * (1 + m/8);
 * e == 0: 2^-6 * m/8 (subnormal).  (e, m) == (15, 7) is NaN.
 * Pins: all 256 codes against the library fp8 dtype; max 448; 126 positive
 * finite non-zero codes; 18 binades. */
double orc_e4m3_value(uint32_t code) {
    int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    v = (e > 0) ? ldexp(1.0 + m / 8.0, e - 7) : ldexp(m / 8.0, -6);
    return s ? -v : v;
}

/* Encode to E4M3 by round-to-nearest-even on its grid.  Magnitudes above the
 * largest finite value saturate to 448: the block-scale quantiser of [P1]
 * "DeepSeek-V4.1", "Check it in numpy", clamps the scale with min(..., 448);
 * the pages never produce the NaN code.  The sign is kept (-0 -> 0x80).
 * Pins: encode(decode(c)) == c for every finite code; agreement with the
 * library fp8 cast on every in-range value tested. */
uint32_t orc_e4m3_encode(float x) {
    uint32_t sign = signbit(x) ? 0x80u : 0u;
    double a = fabs((double)x);
    uint32_t mag;
    if (isnan(x)) return 0x7Fu;
    if (a >= 448.0) {
        mag = 0x7Eu;                                   /* saturate */
    } else if (a < ldexp(1.0, -6)) {
        /* subnormal binade: grid step 2^-9; q == 8 is the smallest normal */
        mag = (uint32_t)rne_int(a / ldexp(1.0, -9));
    } else {
        int ex;
        double fr = frexp(a, &ex);                     /* a = fr * 2^ex, fr in [0.5,1) */
        int e = ex - 1;                                /* a = 2^e * (1 + f) */
        double q = rne_int((fr * 2.0 - 1.0) * 8.0);    /* 3 mantissa bits */
        if (q == 8.0) { e += 1; q = 0.0; }
        mag = (uint32_t)(((e + 7) << 3) | (int)q);     /* a < 448 keeps this <= 0x7E */
    }
    return sign | mag;
}

/* ------------------------------------------------------------------------- */
/* E2M1: [P1] "A Precision Primer", E2M1: eight magnitudes -- one sign bit,
 * two exponent bits, one mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 * no infinity, no NaN.  Bits s|ee|m: e == 0 -> m * 0.5; e > 0 -> 2^(e-1)(1+m/2).
 * Pin: the eight magnitudes printed on the page. */
double orc_e2m1_value(uint32_t nib) {
    int s = (nib >> 3) & 1, e = (nib >> 1) & 3, m = nib & 1;
    double v = (e > 0) ? ldexp(1.0 + m / 2.0, e - 1) : m * 0.5;
    return s ? -v : v;
}

/* Round-to-nearest on the E2M1 ladder ([P1] "DeepSeek-V4.1", "Four bits for
 * the main KV"), ties to the even mantissa (IEEE default; the page's toy
 * breaks ties toward the lower rung, which differs only at exact midpoints),
 * saturating at 6.  Sign kept.
 * Pin: brute-force nearest-rung search with even-code tie-break. */
uint32_t orc_e2m1_encode(float y) {
    uint32_t sign = signbit(y) ? 0x8u : 0u;
    double a = fabs((double)y);
    uint32_t mag;
    if (isnan(y)) return 0x7u;
    if (a >= 6.0) {
        mag = 0x7u;
    } else if (a < 1.0) {
        mag = (uint32_t)rne_int(a * 2.0);              /* 0, 0.5, 1.0 (code 2) */
    } else {
        int ex;
        double fr = frexp(a, &ex);
        int e = ex - 1;                                /* 0, 1 or 2 */
        double q = rne_int((fr * 2.0 - 1.0) * 2.0);    /* 1 mantissa bit */
        if (q == 2.0) { e += 1; q = 0.0; }
        mag = (uint32_t)(((e + 1) << 1) | (int)q);
        if (mag > 7u) mag = 7u;
    }
    return sign | mag;
}

/* ------------------------------------------------------------------------- */
/* bfloat16: the top 16 bits of an fp32, reached by round-to-nearest-even.
 * The bf16 RoPE channels of the V3.2 row ([P1] "DeepSeek-V3.2", "What it
 * costs and what it saves") and the window entries use it.
 * Pin: the library bf16 cast. */
uint32_t orc_bf16_encode(float x) {
    uint32_t u, lo, hi_trunc;
    memcpy(&u, &x, 4);
    if (isnan(x)) return 0x7FC0u;
    hi_trunc = u >> 16;
    lo = u & 0xFFFFu;
    if (lo > 0x8000u) return (hi_trunc + 1u) & 0xFFFFu;
    if (lo < 0x8000u) return hi_trunc;
    return (hi_trunc & 1u) ? ((hi_trunc + 1u) & 0xFFFFu) : hi_trunc;
}

float orc_bf16_value(uint32_t h) {
    uint32_t u = (h & 0xFFFFu) << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static void put_f32(uint8_t* p, float f) { memcpy(p, &f, 4); }
static float get_f32(const uint8_t* p) { float f; memcpy(&f, p, 4); return f; }
static void put_u16(uint8_t* p, uint32_t h) { p[0] = (uint8_t)(h & 0xFF); p[1] = (uint8_t)((h >> 8) & 0xFF); }
static uint32_t get_u16(const uint8_t* p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8); }

/* ------------------------------------------------------------------------- */
/* E8M0 and the MXFP4 block scale ([P1] "DeepSeek-V4", "The indexer in four
 * bits" and [P4] "FP4 main KV: smaller cells": V4's indexer keys and queries
 * use the OCP MXFP4 format, 128 four-bit values plus four E8M0 scales = 68 B).
 * An E8M0 code e is the power of two 2^(e - 127); 0xFF is NaN.  The pages do
 * not state how the shared scale is chosen; the reading taken is the OCP
 * microscaling rule: X = 2^(floor(log2(amax)) - 2), 2 being the exponent of
 * E2M1's largest value 6, clamped to the codes 0 .. 254; a block of zeros
 * takes code 0.  Elements are E2M1(x / X), round-to-nearest-even on the
 * ladder, saturating at 6 (amax / X lies in [4, 8), so values over 6X clamp).
 * Pins: codes 127 -> 1, 128 -> 2, 0 -> 2^-127, 254 -> 2^127; amax 6 -> X = 1,
 * amax 1 -> X = 1/4; blocks on the grid round-trip; |x - x^| <= X below 6X. */
double orc_e8m0_value(uint32_t code) {
    code &= 0xFFu;
    if (code == 0xFFu) return NAN;
    return ldexp(1.0, (int)code - 127);
}

uint32_t orc_mx_scale(float amax) {
    int e;
    if (!(amax > 0.0f)) return 0u;
    (void)frexpf(amax, &e);                 /* amax = m * 2^e, m in [0.5, 1): floor(log2) = e - 1 */
    e = (e - 1) - 2 + 127;
    if (e < 0) e = 0;
    if (e > 254) e = 254;
    return (uint32_t)e;
}

/* The MXFP8 block scale of V4.1's window entry ([P1] "DeepSeek-V4.1", the
 * 528-byte window entry: 512 E4M3 values plus 16 E8M0 scales, one per 32
 * channels).  The same OCP rule with E4M3's largest exponent: X =
 * 2^(floor(log2(amax)) - 8), 8 being the exponent of 448, clamped to the codes
 * 0 .. 254; a block of zeros takes code 0.  Elements are E4M3(x / X),
 * round-to-nearest-even, saturating at 448 (amax / X lies in [256, 512)).
 * Pins: amax 448 -> code 127, amax 1 -> 119; hand-encoded elements; 528 B. */
uint32_t orc_mx8_scale(float amax) {
    int e;
    if (!(amax > 0.0f)) return 0u;
    (void)frexpf(amax, &e);                 /* floor(log2 amax) = e - 1 */
    e = (e - 1) - 8 + 127;
    if (e < 0) e = 0;
    if (e > 254) e = 254;
    return (uint32_t)e;
}

/* ------------------------------------------------------------------------- */
/* Row layouts.
 *  F32        : (dim+rope) fp32                                   c1: 320 / 128 B
 *  BF16       : (dim+rope) bf16                                   c2: 1152 / 256 B
 *  E4M3_S128  : dim E4M3 codes | dim/128 fp32 scales | rope bf16  656 / 132 B
 *               ([P1] "DeepSeek-V3.2", "What it costs and what it saves":
 *               512 B of FP8 latent, four FP32 scales, 64 bf16 RoPE channels;
 *               the indexer key is 128 FP8 bytes plus a 4-byte scale)
 *  E2M1_S16   : dim/2 bytes of nibbles (channel 2i in the low nibble of byte i)
 *               | dim/16 E4M3 scale bytes; no separate RoPE part
 *               ([P1] "DeepSeek-V4.1", "Four bits for the main KV": 256 + 32 =
 *               288 B; [P3] section 3: the indexer key in the same format is
 *               72 B)
 *  MXFP8      : dim E4M3 codes | dim/32 E8M0 scale bytes; no RoPE part (the
 *               window entry: 512 + 16 = 528 B, [P1] "DeepSeek-V4.1")
 *  MXFP4      : dim/2 bytes of nibbles (as E2M1_S16) | dim/32 E8M0 scale bytes;
 *               no RoPE part ([P1] "DeepSeek-V4", "The indexer in four bits":
 *               64 + 4 = 68 B for the 128-channel indexer key)
 * Pins: 656 / 132 / 288 / 72 / 68; 61 x (656 + 132) = 48,068 ([P1]
 * "DeepSeek-V3.2"); 2.5 x (288 + 68) = 890 ([P3], [P4]).
 */
int64_t orc_row_bytes(int fmt, int dim, int rope) {
    if (dim <= 0 || rope < 0) return -1;
    switch (fmt) {
    case ORC_F32: return 4LL * (dim + rope);
    case ORC_BF16: return 2LL * (dim + rope);
    case ORC_E4M3_S128:
        if (dim % 128) return -1;
        return (int64_t)dim + 4LL * (dim / 128) + 2LL * rope;
    case ORC_E2M1_S16:
        if (dim % 16 || rope != 0) return -1;
        return (int64_t)dim / 2 + dim / 16;
    case ORC_MXFP4:
        if (dim % 32 || rope != 0) return -1;
        return (int64_t)dim / 2 + dim / 32;
    case ORC_MXFP8:
        if (dim % 32 || rope != 0) return -1;
        return (int64_t)dim + dim / 32;
    default: return -1;
    }
}

/* Quantise one row of dim+rope fp32 values.
 * E4M3_S128 block of 128 channels: a = max|x| (fp32); s = a / 448 (fp32
 *   division); code_i = E4M3(x_i / s) (fp32 division, then RNE, saturating);
 *   a == 0 gives s = 0 and all codes +0.  The pages state the 656-byte layout
 *   with four fp32 scales but not the scale rule; amax/448 is the plainest one
 *   that maps the block's largest magnitude onto the format's largest value.
 * E2M1_S16 block of 16 channels ([P1] "DeepSeek-V4.1", "Check it in numpy":
 *   the scale maps the block maximum onto 6.0 and is itself an E4M3 value):
 *   s = E4M3(max|x| / 6) (fp32 division, RNE, saturating); if s decodes to 0
 *   every code is +0; else code_i = E2M1(x_i / s_f) with fp32 division.
 * Pins: the page's FP4 worked example (max |latent| 3.861, rel-L2 0.0912);
 *   |x - x^| <= s_f on unclipped FP4 elements; FP8 relative error <= 2^-4. */
int orc_quant_row(int fmt, int dim, int rope, const float* x, uint8_t* row) {
    int64_t nb = orc_row_bytes(fmt, dim, rope);
    int c, b, r;
    if (nb < 0) return -1;
    switch (fmt) {
    case ORC_F32:
        for (c = 0; c < dim + rope; c++) put_f32(row + 4 * c, x[c]);
        return 0;
    case ORC_BF16:
        for (c = 0; c < dim + rope; c++) put_u16(row + 2 * c, orc_bf16_encode(x[c]));
        return 0;
    case ORC_E4M3_S128:
        for (b = 0; b < dim / 128; b++) {
            float a = 0.0f, s;
            for (c = 128 * b; c < 128 * (b + 1); c++) {
                float m = fabsf(x[c]);
                if (m > a) a = m;
            }
            s = a / 448.0f;
            for (c = 128 * b; c < 128 * (b + 1); c++) {
                if (a == 0.0f) { row[c] = 0; continue; }
                row[c] = (uint8_t)orc_e4m3_encode(x[c] / s);
            }
            put_f32(row + dim + 4 * b, s);
        }
        for (r = 0; r < rope; r++)
            put_u16(row + dim + 4 * (dim / 128) + 2 * r, orc_bf16_encode(x[dim + r]));
        return 0;
    case ORC_E2M1_S16:
        memset(row, 0, (size_t)nb);
        for (b = 0; b < dim / 16; b++) {
            float a = 0.0f, sf;
            uint32_t sc;
            for (c = 16 * b; c < 16 * (b + 1); c++) {
                float m = fabsf(x[c]);
                if (m > a) a = m;
            }
            sc = orc_e4m3_encode(a / 6.0f);
            sf = (float)orc_e4m3_value(sc);
            row[dim / 2 + b] = (uint8_t)sc;
            for (c = 16 * b; c < 16 * (b + 1); c++) {
                uint32_t nib = (sf == 0.0f) ? 0u : orc_e2m1_encode(x[c] / sf);
                row[c / 2] |= (uint8_t)((c & 1) ? (nib << 4) : nib);
            }
        }
        return 0;
    case ORC_MXFP8:
        for (b = 0; b < dim / 32; b++) {
            float a = 0.0f, X;
            uint32_t sc;
            for (c = 32 * b; c < 32 * (b + 1); c++) {
                float m = fabsf(x[c]);
                if (m > a) a = m;
            }
            sc = orc_mx8_scale(a);
            X = ldexpf(1.0f, (int)sc - 127);         /* exact, 2^-127 as an fp32 subnormal */
            row[dim + b] = (uint8_t)sc;
            for (c = 32 * b; c < 32 * (b + 1); c++) row[c] = (uint8_t)((a == 0.0f) ? 0u : orc_e4m3_encode(x[c] / X));
        }
        return 0;
    case ORC_MXFP4:
        memset(row, 0, (size_t)nb);
        for (b = 0; b < dim / 32; b++) {
            float a = 0.0f, X;
            uint32_t sc;
            for (c = 32 * b; c < 32 * (b + 1); c++) {
                float m = fabsf(x[c]);
                if (m > a) a = m;
            }
            sc = orc_mx_scale(a);
            X = ldexpf(1.0f, (int)sc - 127);         /* exact, 2^-127 as an fp32 subnormal */
            row[dim / 2 + b] = (uint8_t)sc;
            for (c = 32 * b; c < 32 * (b + 1); c++) {
                uint32_t nib = (a == 0.0f) ? 0u : orc_e2m1_encode(x[c] / X);
                row[c / 2] |= (uint8_t)((c & 1) ? (nib << 4) : nib);
            }
        }
        return 0;
    }
    return -1;
}

/* Dequantise one row to the exact values it encodes (in double):
 * E4M3 code x fp32 scale (exact: 4 x 24 significant bits), bf16 RoPE as is,
 * E2M1 x E4M3 scale (exact). */
int orc_dequant_row(int fmt, int dim, int rope, const uint8_t* row, double* out) {
    int c;
    if (orc_row_bytes(fmt, dim, rope) < 0) return -1;
    switch (fmt) {
    case ORC_F32:
        for (c = 0; c < dim + rope; c++) out[c] = (double)get_f32(row + 4 * c);
        return 0;
    case ORC_BF16:
        for (c = 0; c < dim + rope; c++) out[c] = (double)orc_bf16_value(get_u16(row + 2 * c));
        return 0;
    case ORC_E4M3_S128:
        for (c = 0; c < dim; c++)
            out[c] = orc_e4m3_value(row[c]) * (double)get_f32(row + dim + 4 * (c / 128));
        for (c = 0; c < rope; c++)
            out[dim + c] = (double)orc_bf16_value(get_u16(row + dim + 4 * (dim / 128) + 2 * c));
        return 0;
    case ORC_E2M1_S16:
        for (c = 0; c < dim; c++) {
            uint32_t nib = (c & 1) ? (row[c / 2] >> 4) : (row[c / 2] & 0xF);
            out[c] = orc_e2m1_value(nib) * orc_e4m3_value(row[dim / 2 + c / 16]);
        }
        return 0;
    case ORC_MXFP8:
        for (c = 0; c < dim; c++) out[c] = orc_e4m3_value(row[c]) * orc_e8m0_value(row[dim + c / 32]);
        return 0;
    case ORC_MXFP4:
        for (c = 0; c < dim; c++) {
            uint32_t nib = (c & 1) ? (row[c / 2] >> 4) : (row[c / 2] & 0xF);
            out[c] = orc_e2m1_value(nib) * orc_e8m0_value(row[dim / 2 + c / 32]);
        }
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------------------- */
/* Append one decode step's entries.  The main entry is the [c_KV ; k_R] vector
 * the absorbed kernels read ([P1] "DeepSeek-V2", "Why RoPE breaks the trick";
 * [P2] Part 2 "What replaced MLA"), quantised after RoPE ([P1] "DeepSeek-V4.1",
 * "Four bits for the main KV").  The indexer key is quantised the same way.
 * The window entry goes to ring slot pos mod W ([P1] "Sliding Window
 * Attention", "Definition and the bounded cache") as bf16.
 * Any of main / indexer / window may be absent (NULL). */
int orc_append(int main_fmt, int main_dim, int main_rope, int idx_fmt, int idx_dim,
               const float* new_main, const float* new_idx, const int32_t* slots,
               int B, int n_new, int64_t capacity,
               uint8_t* main_cache, int64_t main_seq_stride,
               uint8_t* idx_cache, int64_t idx_seq_stride,
               const float* new_win, const int32_t* win_pos,
               uint16_t* win_ring, int W, int Dw) {
    int b, i, c;
    int64_t mb = main_cache ? orc_row_bytes(main_fmt, main_dim, main_rope) : 0;
    int64_t ib = idx_cache ? orc_row_bytes(idx_fmt, idx_dim, 0) : 0;
    if (B < 0 || n_new < 0 || mb < 0 || ib < 0) return -1;
    for (b = 0; b < B; b++)
        for (i = 0; i < n_new; i++) {
            int64_t slot = slots[(int64_t)b * n_new + i];
            if ((main_cache || idx_cache) && (slot < 0 || slot >= capacity)) return -2;
        }
    for (b = 0; b < B; b++) {
#pragma omp parallel for schedule(static)
        for (i = 0; i < n_new; i++) {
            int64_t slot;
            if (!main_cache && !idx_cache) continue;
            slot = slots[(int64_t)b * n_new + i];
            if (main_cache)
                orc_quant_row(main_fmt, main_dim, main_rope,
                              new_main + ((int64_t)b * n_new + i) * (main_dim + main_rope),
                              main_cache + b * main_seq_stride + slot * mb);
            if (idx_cache)
                orc_quant_row(idx_fmt, idx_dim, 0, new_idx + ((int64_t)b * n_new + i) * idx_dim,
                              idx_cache + b * idx_seq_stride + slot * ib);
        }
        if (win_ring) {
            int pos = win_pos[b];
            if (pos < 0 || W <= 0) return -3;
            for (c = 0; c < Dw; c++)
                win_ring[((int64_t)b * W + pos % W) * Dw + c] =
                    (uint16_t)orc_bf16_encode(new_win[(int64_t)b * Dw + c]);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Lightning-indexer score ([P1] "DeepSeek-V3.2", "The lightning indexer",
 * eq. 1; [P2] Part 1 "The indexer"):
 *     I[b,s] = sum_j w[b,j] * ReLU(sigma * q_idx[b,j] . k_idx[b,s])
 * with one shared indexer key per cached row, sigma = d_I^-0.5 applied
 * inside the ReLU and the per-head weights pre-scaled by the caller (x H_I^-0.5
 * in the V3.2 code).  Rows at or beyond n_visible[b] are causally masked to
 * -inf before selection ([P2] Part 1: the mask is added before top-k; [P2]
 * "HCA": entry e is visible iff e < (p+1) // m).
 * With a candidate pool (cand != NULL, [P4] "The Hierarchical Sparse
 * Indexer"), score i of row b is that of position cand[b,i] (-inf when the
 * position is negative or not visible) and scores is [B, n_cand].
 * q_idx holds the exact values of the bf16 queries, [B, H_I, idx_dim].  With
 * MXFP4 keys the query is quantised the same way first (each head's vector as
 * an MXFP4 row): V4 caches, loads and multiplies the indexer's query-key path
 * entirely in FP4 ([P1] "DeepSeek-V4", "The indexer in four bits").
 * Pins: single-head and one-hot-weight cases reduce to a dot product;
 * I(q) - I(-q) is the plain bilinear form sum_j w_j sigma q_j.k; ReLU votes
 * are non-negative; brute force on the tiny case. */
int orc_indexer_scores(int idx_fmt, int idx_dim, const float* q_idx, const float* w, float sigma,
                       const uint8_t* idx_cache, int64_t idx_seq_stride, const int32_t* n_visible,
                       const int32_t* cand, int n_cand,
                       int B, int H_I, int64_t n_rows, float* scores) {
    int64_t rb = orc_row_bytes(idx_fmt, idx_dim, 0);
    int64_t n_out = cand ? (int64_t)n_cand : n_rows;
    int b;
    if (rb < 0 || B < 0 || H_I <= 0 || n_rows < 0) return -1;
    for (b = 0; b < B; b++) {
        int64_t i;
        int j0;
        double* qd = (double*)malloc(sizeof(double) * (size_t)H_I * idx_dim);
        if (n_visible[b] < 0 || n_visible[b] > n_rows) {
            free(qd);
            return -2;
        }
        for (j0 = 0; j0 < H_I; j0++) {                 /* the queries the scores use */
            const float* qj = q_idx + ((int64_t)b * H_I + j0) * idx_dim;
            int c;
            if (idx_fmt == ORC_MXFP4) {
                uint8_t* qrow = (uint8_t*)malloc((size_t)rb);
                orc_quant_row(ORC_MXFP4, idx_dim, 0, qj, qrow);
                orc_dequant_row(ORC_MXFP4, idx_dim, 0, qrow, qd + (int64_t)j0 * idx_dim);
                free(qrow);
            } else {
                for (c = 0; c < idx_dim; c++) qd[(int64_t)j0 * idx_dim + c] = (double)qj[c];
            }
        }
#pragma omp parallel for schedule(static)
        for (i = 0; i < n_out; i++) {
            double* k = (double*)malloc(sizeof(double) * idx_dim);
            int64_t s = cand ? (int64_t)cand[(int64_t)b * n_cand + i] : i;
            double acc = 0.0;
            int j, c;
            if (s < 0 || s >= n_visible[b]) {
                scores[b * n_out + i] = -INFINITY;
                free(k);
                continue;
            }
            orc_dequant_row(idx_fmt, idx_dim, 0, idx_cache + b * idx_seq_stride + s * rb, k);
            for (j = 0; j < H_I; j++) {
                const double* qj = qd + (int64_t)j * idx_dim;
                double d = 0.0, v;
                for (c = 0; c < idx_dim; c++) d += qj[c] * k[c];
                v = (double)sigma * d;
                if (v < 0.0) v = 0.0;                          /* ReLU */
                acc += (double)w[(int64_t)b * H_I + j] * v;
            }
            scores[b * n_out + i] = (float)acc;
            free(k);
        }
        free(qd);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Top-k ([P1] "DeepSeek-V3.2", eq. 2; [P2] Part 1 "The indexer": topk over the
 * masked scores, int32 indices).  Visible positions are ordered by score
 * descending, then position ascending; the first min(k, n_visible) are kept
 * and the remaining slots hold -1 ([P2] "CSA: two changes to HCA": the -1
 * sentinel for slots with no legal entry).
 * Pins: brute-force sort on tiny cases; k >= n_visible selects every visible
 * position; the -1 count. */
typedef struct { float score; int32_t pos; } orc_pair;

static int cmp_pair(const void* pa, const void* pb) {
    const orc_pair* a = (const orc_pair*)pa;
    const orc_pair* b = (const orc_pair*)pb;
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
    return (a->pos < b->pos) ? -1 : (a->pos > b->pos);
}

int orc_topk(const float* scores, int64_t n_rows, const int32_t* n_visible,
             const int32_t* cand, int n_cand, int B, int k, int32_t* out_idx) {
    int64_t n_in = cand ? (int64_t)n_cand : n_rows;
    int b;
    if (B < 0 || k < 0 || n_rows < 0) return -1;
    for (b = 0; b < B; b++) {
        orc_pair* v = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)(n_in > 0 ? n_in : 1));
        int64_t n = 0, i;
        for (i = 0; i < n_in; i++) {
            int64_t s = cand ? (int64_t)cand[(int64_t)b * n_cand + i] : i;
            if (s < 0 || s >= n_visible[b]) continue;
            v[n].score = scores[b * n_in + i];
            v[n].pos = (int32_t)s;
            n++;
        }
        qsort(v, (size_t)n, sizeof(orc_pair), cmp_pair);
        for (i = 0; i < k; i++) out_idx[(int64_t)b * k + i] = (i < n) ? v[i].pos : -1;
        free(v);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Candidate pool of the hierarchical sparse indexer ([P4] "The Hierarchical
 * Sparse Indexer: bounded sweeps"; [P1] "DeepSeek-V4.1", "The hierarchical
 * indexer"): the
 * positions of one layer's scores are grouped into blocks of `block`
 * consecutive positions (block i = positions block*i .. block*i + block - 1),
 * each block is scored by the largest score among its visible positions
 * (blocks with none are left out), and the n_blocks best blocks are kept,
 * ordered by that score descending, then block index ascending (the same
 * order as the top-k).  out_blocks[b, :] holds their block indices, -1 past
 * the number of blocks with a visible position.
 * Pins: block 1 reduces to the top-k; enough blocks keep every block with a
 * visible position; the pool holds every position of the layer's own top-k
 * for k <= n_blocks (a block holding the j-th best position scores at least
 * as much, and at most j - 1 other blocks score more); ties go to the smaller
 * block; hand fixtures. */
int orc_pool(const float* scores, int64_t n_rows, const int32_t* n_visible, int B, int block, int n_blocks,
             int32_t* out_blocks) {
    int b;
    if (B < 0 || block <= 0 || n_blocks < 0 || n_rows < 0) return -1;
    for (b = 0; b < B; b++) {
        int64_t nb = (n_rows + block - 1) / block, n = 0, i;
        orc_pair* v = (orc_pair*)malloc(sizeof(orc_pair) * (size_t)(nb > 0 ? nb : 1));
        if (n_visible[b] < 0 || n_visible[b] > n_rows) {
            free(v);
            return -2;
        }
        for (i = 0; i < nb; i++) {
            int64_t s, lo = i * block, hi = lo + block;
            int any = 0;
            float m = 0.0f;
            if (hi > n_visible[b]) hi = n_visible[b];
            for (s = lo; s < hi; s++) {
                float x = scores[b * n_rows + s];
                if (!any || x > m) m = x;
                any = 1;
            }
            if (!any) continue;
            v[n].score = m;
            v[n].pos = (int32_t)i;
            n++;
        }
        qsort(v, (size_t)n, sizeof(orc_pair), cmp_pair);
        for (i = 0; i < n_blocks; i++) out_blocks[(int64_t)b * n_blocks + i] = (i < n) ? v[i].pos : -1;
        free(v);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Sparse attention in the absorbed (MQA) form ([P1] "DeepSeek-V2", "Why RoPE
 * breaks the trick" and "Check it in numpy"; [P2] Part 2 "What replaced MLA";
 * [P1] "DeepSeek-V3.2": each selected latent is shared by all query heads).
 * For each (b, h), U = the selected rows (idx != -1) plus window slots
 * 0 .. win_len[b]-1 (the window is concatenated with the selected entries,
 * [P1] "DeepSeek-V4", "A window in every layer"; not de-duplicated):
 *   z_u  = softmax_scale * q[b,h,:] . K_u          (K_u: all dim+rope channels)
 *   lse  = max z + ln sum_u exp(z_u - max z)       (natural log, scale included)
 *   o[c] = sum_u exp(z_u - lse) * K_u[c],  c < d_v  (V = the leading d_v channels:
 *          the 512 latent channels for V3.2, the whole row when K = V)
 * An empty U gives lse = -inf and o = 0.
 * With attention sinks ([P2] Part 2 "The sliding window", "Attention sinks":
 * one learned scalar per head is appended to each row of scaled scores as an
 * extra column before the softmax and dropped after it; the column has no
 * value vector), sinks[h] joins the normaliser only:
 *   lse  = log(sum_u exp(z_u) + exp(sinks[h])),  o[c] = sum_u exp(z_u - lse) * K_u[c]
 * so the weights of U sum to 1 - p_sink; an empty U gives lse = sinks[h], o = 0.
 * sinks == NULL (or -inf) is the plain softmax.
 * O-RoPE ([P2] Part 2 "What replaced MLA", "Partial RoPE, and its inverse on
 * the output": K = V carries the rotation of its trailing RoPE channels, and
 * V4 undoes it on the output at the query position, apply_rotary_pos_emb(o,
 * cos, -sin)): with rope_dim > 0 the trailing rope_dim output channels, as
 * halves x1 = o[d_v - rope_dim .. d_v - rope_dim/2), x2 = the rest (the
 * rotate-half pairing of that function), become x1 cos + x2 sin and
 * x2 cos - x1 sin, with (cos, sin) = rope_cs[b, i] for pair i.
 * Window rows are bf16, [B, W, dim+rope].
 * Pins: absorbed = naive MLA with explicit up-projections; k >= visible rows
 * equals dense softmax attention; LSE merge of any partition equals the whole;
 * window-only equals dense attention over the window. */
int orc_attention(int main_fmt, int main_dim, int main_rope, int d_v,
                  const float* q, const uint8_t* main_cache, int64_t main_seq_stride, int64_t capacity,
                  const int32_t* idx, int k,
                  const uint16_t* win_ring, const int32_t* win_len, int W,
                  float softmax_scale, const float* sinks, int rope_dim, const float* rope_cs,
                  int B, int H, float* out, float* lse) {
    int D = main_dim + main_rope;
    int64_t rb = orc_row_bytes(main_fmt, main_dim, main_rope);
    int b;
    if (rb < 0 || d_v <= 0 || d_v > D || B < 0 || H <= 0 || k < 0) return -1;
    if (rope_dim < 0 || rope_dim % 2 || rope_dim > d_v || (rope_dim > 0 && !rope_cs)) return -1;
    for (b = 0; b < B; b++) {
        int i, nw = 0, nu = 0;
        for (i = 0; i < k; i++) {
            int32_t s = idx[(int64_t)b * k + i];
            if (s < -1 || s >= capacity) return -2;
        }
        if (win_ring) {
            nw = win_len[b];
            if (nw < 0 || nw > W) return -3;
        }
        for (i = 0; i < k; i++) nu += (idx[(int64_t)b * k + i] >= 0);
        nu += nw;
        {
            /* the gathered, dequantised rows of U, [nu, D] */
            double* rows = (double*)malloc(sizeof(double) * (size_t)(nu > 0 ? nu : 1) * D);
            int u = 0, h;
            for (i = 0; i < k; i++) {
                int32_t s = idx[(int64_t)b * k + i];
                if (s < 0) continue;
                orc_dequant_row(main_fmt, main_dim, main_rope,
                                main_cache + b * main_seq_stride + (int64_t)s * rb, rows + (int64_t)u * D);
                u++;
            }
            for (i = 0; i < nw; i++, u++) {
                int c;
                for (c = 0; c < D; c++)
                    rows[(int64_t)u * D + c] =
                        (double)orc_bf16_value(win_ring[((int64_t)b * W + i) * D + c]);
            }
#pragma omp parallel for schedule(static)
            for (h = 0; h < H; h++) {
                const float* qh = q + ((int64_t)b * H + h) * D;
                double* z = (double*)malloc(sizeof(double) * (size_t)(nu > 0 ? nu : 1));
                double m = -INFINITY, sum = 0.0, l;
                double sk = sinks ? (double)sinks[h] : -INFINITY;   /* the sink column's logit */
                int uu, c;
                for (uu = 0; uu < nu; uu++) {
                    double d = 0.0;
                    for (c = 0; c < D; c++) d += (double)qh[c] * rows[(int64_t)uu * D + c];
                    z[uu] = (double)softmax_scale * d;
                    if (z[uu] > m) m = z[uu];
                }
                if (sk > m) m = sk;
                if (m == -INFINITY) {
                    lse[(int64_t)b * H + h] = -INFINITY;
                    for (c = 0; c < d_v; c++) out[((int64_t)b * H + h) * d_v + c] = 0.0f;
                    free(z);
                    continue;
                }
                for (uu = 0; uu < nu; uu++) sum += exp(z[uu] - m);
                if (sk > -INFINITY) sum += exp(sk - m);
                l = m + log(sum);
                lse[(int64_t)b * H + h] = (float)l;
                {
                    double* ov = (double*)malloc(sizeof(double) * (size_t)d_v);
                    int hr = rope_dim / 2, ii;
                    for (c = 0; c < d_v; c++) {
                        double o = 0.0;
                        for (uu = 0; uu < nu; uu++) o += exp(z[uu] - l) * rows[(int64_t)uu * D + c];
                        ov[c] = o;
                    }
                    for (ii = 0; ii < hr; ii++) {            /* un-rotate pair ii at the query position */
                        double cs = rope_cs[((int64_t)b * hr + ii) * 2], sn = rope_cs[((int64_t)b * hr + ii) * 2 + 1];
                        double x1 = ov[d_v - rope_dim + ii], x2 = ov[d_v - hr + ii];
                        ov[d_v - rope_dim + ii] = x1 * cs + x2 * sn;
                        ov[d_v - hr + ii] = x2 * cs - x1 * sn;
                    }
                    for (c = 0; c < d_v; c++) out[((int64_t)b * H + h) * d_v + c] = (float)ov[c];
                    free(ov);
                }
                free(z);
            }
            free(rows);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Element-wise batch forms of the scalar codecs, for the tests. */
void orc_e4m3_encode_n(const float* x, int64_t n, uint8_t* out) {
    int64_t i;
    for (i = 0; i < n; i++) out[i] = (uint8_t)orc_e4m3_encode(x[i]);
}
void orc_e2m1_encode_n(const float* x, int64_t n, uint8_t* out) {
    int64_t i;
    for (i = 0; i < n; i++) out[i] = (uint8_t)orc_e2m1_encode(x[i]);
}
void orc_bf16_encode_n(const float* x, int64_t n, uint16_t* out) {
    int64_t i;
    for (i = 0; i < n; i++) out[i] = (uint16_t)orc_bf16_encode(x[i]);
}

/* ------------------------------------------------------------------------- */
/* The CSA2 compressor at append ([P1] "DeepSeek-V4.1", "CSA2: the simplified
 * compressor": windows of m tokens that do not overlap and no position bias;
 * [P2] Part 2, the compressor's training-path code: a softmax of the gate over
 * the window's m tokens per channel, the gated sum of the kv vectors, then the
 * kv normalisation).  For each sequence b, from the already projected kv[b, i, c]
 * and gate[b, i, c] (i < m, c < D):
 *     w[i, c]   = exp(gate[i, c]) / sum_j exp(gate[j, c])
 *     p[c]      = sum_i w[i, c] kv[i, c]
 *     y[c]      = p[c] / sqrt(mean_c p[c]^2 + eps) * g[c]       (RMS normalisation)
 * and, with rope_dim r > 0, the trailing r channels rotated forward at the
 * window's position in the rotate-half pairing: x1 = y[D-r .. D-r/2),
 * x2 = y[D-r/2 .. D): (x1 cos - x2 sin, x2 cos + x1 sin), (cos, sin) =
 * rope_cs[b, i].  The normalisation is read as RMSNorm with a weight (the
 * pages name kv_norm only); g == NULL means ones.  Output fp32 [B, D] (the
 * fp64 result rounded).  Pins: m = 1 is the normalised kv; equal gates give
 * the normalised mean (the mean-of-pairs stand-in at m = 2); a dominant gate
 * selects its token; the weights sum to one; the rotation keeps pair norms and
 * the output RoPE inverse undoes it. */
int orc_compress(int D, int m, const float* kv, const float* gate, const float* g, double eps, int rope_dim,
                 const float* rope_cs, int B, float* out) {
    if (D <= 0 || m <= 0 || B < 0 || rope_dim < 0 || rope_dim > D || rope_dim % 2) return -1;
    double* p = (double*)malloc(sizeof(double) * (size_t)D);
    if (!p) return -2;
    for (int b = 0; b < B; b++) {
        const float* K = kv + (int64_t)b * m * D;
        const float* G = gate + (int64_t)b * m * D;
        double ss = 0.0;
        for (int c = 0; c < D; c++) {
            double mx = -INFINITY, den = 0.0, num = 0.0;
            for (int i = 0; i < m; i++)
                if ((double)G[(int64_t)i * D + c] > mx) mx = G[(int64_t)i * D + c];
            for (int i = 0; i < m; i++) {
                double e = exp((double)G[(int64_t)i * D + c] - mx);
                den += e;
                num += e * (double)K[(int64_t)i * D + c];
            }
            p[c] = num / den;
            ss += p[c] * p[c];
        }
        const double inv = 1.0 / sqrt(ss / D + eps);
        for (int c = 0; c < D; c++) p[c] = p[c] * inv * (g ? (double)g[c] : 1.0);
        const int h = rope_dim / 2;
        for (int i = 0; i < h; i++) {
            const double cs = rope_cs[((int64_t)b * h + i) * 2], sn = rope_cs[((int64_t)b * h + i) * 2 + 1];
            const double x1 = p[D - rope_dim + i], x2 = p[D - h + i];
            p[D - rope_dim + i] = x1 * cs - x2 * sn;
            p[D - h + i] = x2 * cs + x1 * sn;
        }
        for (int c = 0; c < D; c++) out[(int64_t)b * D + c] = (float)p[c];
    }
    free(p);
    return 0;
}
