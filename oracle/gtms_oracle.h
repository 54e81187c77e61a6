/*
 * Oracle for the grouped tril mask softmax: TEST INFRASTRUCTURE ONLY.
 *
 * Declarations of the plain fp64 CPU oracle in gtms_oracle.c. Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load this library. The GPU product
 * library neither includes this header nor links the oracle, and the oracle includes
 * nothing of the product.
 *
 * Element-type codes: 0 = IEEE binary32, 1 = IEEE binary16, 2 = bfloat16.
 * Status codes: 0 = ok, 1 = invalid argument, 2 = unknown element type.
 */
#ifndef GTMS_ORACLE_H
#define GTMS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Full tensor: in and out are host arrays of B*M*S*S elements, row-major [B, M, S, S];
 * seq_lens holds B raw lengths (clamped to [0, S]). out receives fp64 results. */
int gtms_oracle_f64(const void* in, double* out, const int32_t* seq_lens, int64_t B,
                    int64_t M, int64_t S, float scale, int dtype);

/* Same, with every result rounded to nearest-even into the input's element type. */
int gtms_oracle(const void* in, void* out, const int32_t* seq_lens, int64_t B, int64_t M,
                int64_t S, float scale, int dtype);

/* Independent rows: rows_in holds nrows rows of S elements; row i is row index row[i] of a
 * plane whose batch has raw length seq_len[i]. rows_out receives nrows*S fp64 results. */
int gtms_oracle_rows_f64(const void* rows_in, double* rows_out, const int64_t* row,
                         const int32_t* seq_len, int64_t nrows, int64_t S, float scale,
                         int dtype);

/* Backward of the same operation: given the forward output Y and an upstream gradient dY
 * (both [B, M, S, S] in the element type), write dX in fp64. */
int gtms_oracle_backward_f64(const void* y, const void* dy, double* dx,
                             const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                             float scale, int dtype);

/* Backward of independent rows: y_rows and dy_rows hold nrows rows of S elements; row i is
 * row index row[i] of a plane whose batch has raw length seq_len[i]. dx_rows receives
 * nrows*S fp64 results. */
int gtms_oracle_backward_rows_f64(const void* y_rows, const void* dy_rows, double* dx_rows,
                                  const int64_t* row, const int32_t* seq_len, int64_t nrows,
                                  int64_t S, float scale, int dtype);

/* Mask variants (ScaledMaskSoftmax article, sections 2.1, 4.1 and 6). A row's softmax runs
 * over its kept elements only; a row with no kept element is all zeros. seq_lens may be
 * NULL, meaning every valid length is S; otherwise element (r, c) needs r < L_b and c < L_b.
 *
 * Band: element (r, c) is kept when lo <= c - r <= hi (besides the length condition).
 * Masked: element (b, m, r, c) is kept when mask[b*mask_sb + m*mask_sm + r*mask_sr + c] is
 * non-zero (strides in bytes, zero for a broadcast dimension; the column stride is 1). */
int gtms_oracle_band_f64(const void* in, double* out, const int32_t* seq_lens, int64_t B,
                         int64_t M, int64_t S, int64_t lo, int64_t hi, float scale,
                         int dtype);
int gtms_oracle_band_backward_f64(const void* y, const void* dy, double* dx,
                                  const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                                  int64_t lo, int64_t hi, float scale, int dtype);
int gtms_oracle_masked_f64(const void* in, double* out, const uint8_t* mask, int64_t mask_sb,
                           int64_t mask_sm, int64_t mask_sr, const int32_t* seq_lens,
                           int64_t B, int64_t M, int64_t S, float scale, int dtype);
int gtms_oracle_masked_backward_f64(const void* y, const void* dy, double* dx,
                                    const uint8_t* mask, int64_t mask_sb, int64_t mask_sm,
                                    int64_t mask_sr, const int32_t* seq_lens, int64_t B,
                                    int64_t M, int64_t S, float scale, int dtype);

/* Attention with the grouped tril mask (self-attention article, sections 1-2: scores,
 * softmax, weighted sum of values): Q, K, V [B, M, S, D] in the element type; for query row
 * r < L_b, out[r] = sum_{c <= r} softmax_c(scale * Q[r].K[c]) V[c]; rows r >= L_b are zero.
 * out receives B*M*S*D fp64 values. */
int gtms_oracle_attention_f64(const void* q, const void* k, const void* v, double* out,
                              const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                              int64_t D, float scale, int dtype);

/* One query row r of one head: q, k, v point at the head's [S, D] elements; out receives
 * the D fp64 values of row r for a batch of raw valid length seq_len. */
int gtms_oracle_attention_row_f64(const void* q, const void* k, const void* v, double* out,
                                  int64_t r, int32_t seq_len, int64_t S, int64_t D,
                                  float scale, int dtype);

/* The element codec, exported so that it can be pinned on its own. */
double gtms_oracle_decode(uint32_t bits, int dtype);
uint32_t gtms_oracle_encode(double v, int dtype);

#ifdef __cplusplus
}
#endif

#endif
