/*
 * oracle.h -- plain CPU oracle for indexer-selected sparse attention over a
 * block-scaled latent KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this.  It is used by the test suite, the smoke check and the CPU
 * baseline leg of the benchmark.  It shares no code, header, table or helper
 * with the HIP library.
 *
 * Conventions: host pointers only; row bytes are little-endian; all
 * accumulation is in double; every function returns 0 on success and a
 * negative number on a bad argument.
 */
#ifndef ORC_ORACLE_H
#define ORC_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Row formats (value of the `fmt` arguments). */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_E4M3_S128 = 2, ORC_E2M1_S16 = 3, ORC_MXFP4 = 4, ORC_MXFP8 = 5 };

/* Scalar codecs. */
double   orc_e4m3_value(uint32_t code);   /* NaN for 0x7F / 0xFF */
uint32_t orc_e4m3_encode(float x);        /* RNE, saturating at +-448 */
double   orc_e2m1_value(uint32_t nib);
uint32_t orc_e2m1_encode(float y);        /* RNE on the ladder, saturating at +-6 */
uint32_t orc_bf16_encode(float x);        /* RNE */
double   orc_e8m0_value(uint32_t code);   /* 2^(code - 127); NaN for 0xFF */
uint32_t orc_mx_scale(float amax);        /* shared exponent code of an MXFP4 block */
uint32_t orc_mx8_scale(float amax);       /* shared exponent code of an MXFP8 (E4M3) block */
float    orc_bf16_value(uint32_t h);

/* Rows. */
int64_t orc_row_bytes(int fmt, int dim, int rope);
int     orc_quant_row(int fmt, int dim, int rope, const float* x, uint8_t* row);
int     orc_dequant_row(int fmt, int dim, int rope, const uint8_t* row, double* out);

/* Append: quantise new entries into the caches at their slots, write the window ring. */
int orc_append(int main_fmt, int main_dim, int main_rope, int idx_fmt, int idx_dim,
               const float* new_main, const float* new_idx, const int32_t* slots,
               int B, int n_new, int64_t capacity,
               uint8_t* main_cache, int64_t main_seq_stride,
               uint8_t* idx_cache, int64_t idx_seq_stride,
               const float* new_win, const int32_t* win_pos,
               uint16_t* win_ring, int W, int Dw);

/* Lightning-indexer scores, fp32 out, -inf beyond n_visible. */
int orc_indexer_scores(int idx_fmt, int idx_dim, const float* q_idx, const float* w, float sigma,
                       const uint8_t* idx_cache, int64_t idx_seq_stride, const int32_t* n_visible,
                       const int32_t* cand, int n_cand,
                       int B, int H_I, int64_t n_rows, float* scores);

/* Top-k over the visible scores. */
int orc_topk(const float* scores, int64_t n_rows, const int32_t* n_visible,
             const int32_t* cand, int n_cand, int B, int k, int32_t* out_idx);

/* Sparse absorbed-MLA attention over the selected rows plus the window. */
int orc_compress(int D, int m, const float* kv, const float* gate, const float* g, double eps, int rope_dim,
                 const float* rope_cs, int B, float* out);
int orc_attention(int main_fmt, int main_dim, int main_rope, int d_v,
                  const float* q, const uint8_t* main_cache, int64_t main_seq_stride, int64_t capacity,
                  const int32_t* idx, int k,
                  const uint16_t* win_ring, const int32_t* win_len, int W,
                  float softmax_scale, const float* sinks, int rope_dim, const float* rope_cs,
                  int B, int H, float* out, float* lse);

int orc_num_threads(void);

/* Element-wise batch codecs (test helpers). */
void orc_e4m3_encode_n(const float* x, int64_t n, uint8_t* out);
void orc_e2m1_encode_n(const float* x, int64_t n, uint8_t* out);
void orc_bf16_encode_n(const float* x, int64_t n, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
