/*
 * Oracle for the grouped tril mask softmax: TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU implementation in fp64 of what the GPU path
 * computes. Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load it. It shares no code, header, table or helper with the GPU library, and neither
 * side includes or links the other. Single-threaded on purpose.
 *
 * What it computes comes from the page "Fused grouped tril mask softmax"
 * (github aoxy/Attention-Mask-Optimization, README):
 *   - the operator-behaviour section (a torch loop giving the fused computation): X has
 *     shape [B, M, S, S]; every plane of batch b shares one valid length L_b; element
 *     (row, col) is kept when row < L_b, col < L_b and row >= col; kept elements go
 *     through a softmax along the row; the rest are filled with the most negative finite
 *     value before that softmax, so they contribute nothing;
 *   - the three masks printed after that listing (S = 5, lengths 3, 4, 5), which show the
 *     kept set row by row;
 *   - the printed output, whose rows at or beyond L_b and whose upper triangle are zero.
 * The listing finally sets every element equal to 1/S to zero. That step exists only to
 * erase the uniform rows its softmax produces for fully masked rows; here a row with no
 * kept element is written as zeros directly, and a kept element is never zeroed because of
 * its value.
 *
 * The scale factor multiplies the scores before the softmax, as in the page
 * "优化ScaledMaskSoftmax算子" (ScaledMaskSoftmax article), sections 2.1 and 4.1.
 *
 * Readings where the pages are silent:
 *   - seq_lens values are clamped to [0, S] (the listing's predicate tolerates any value);
 *   - results are rounded to nearest, ties to even, into the element type;
 *   - a zero is +0.0;
 *   - NaN or infinity inside a kept prefix propagates by IEEE arithmetic.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "gtms_oracle.h"

enum { OK = 0, ERR_ARG = 1, ERR_DTYPE = 2 };

/* ------------------------------------------------------------------------------------
 * Element codec. A binary floating-point format with `ebits` exponent bits and `pbits`
 * stored fraction bits, exponent bias 2^(ebits-1) - 1 (IEEE 754 layout):
 *   binary32: 8 / 23, binary16: 5 / 10, bfloat16: 8 / 7.
 * ------------------------------------------------------------------------------------ */
static int format_of(int dtype, int* ebits, int* pbits, int* bytes) {
    switch (dtype) {
        case 0: *ebits = 8; *pbits = 23; *bytes = 4; return 1;
        case 1: *ebits = 5; *pbits = 10; *bytes = 2; return 1;
        case 2: *ebits = 8; *pbits = 7; *bytes = 2; return 1;
        default: return 0;
    }
}

static double decode_bits(uint32_t bits, int ebits, int pbits) {
    uint32_t emax = (1u << ebits) - 1;
    int bias = (int)(emax >> 1);
    uint32_t sign = (bits >> (ebits + pbits)) & 1u;
    uint32_t e = (bits >> pbits) & emax;
    uint32_t f = bits & ((1u << pbits) - 1);
    double mag;
    if (e == emax)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, 1 - bias - pbits); /* subnormal: f * 2^(emin - pbits) */
    else
        mag = ldexp((double)(f | (1u << pbits)), (int)e - bias - pbits);
    return sign ? -mag : mag;
}

/* Round v to the nearest representable value, ties to even, and return its bits. */
static uint32_t encode_bits(double v, int ebits, int pbits) {
    uint32_t emax = (1u << ebits) - 1;
    int bias = (int)(emax >> 1);
    int emin = 1 - bias;
    uint32_t sign = signbit(v) ? (1u << (ebits + pbits)) : 0u;
    if (isnan(v)) return sign | (emax << pbits) | (1u << (pbits - 1));
    double a = fabs(v);
    if (isinf(a)) return sign | (emax << pbits);
    if (a == 0.0) return sign;
    int E;
    frexp(a, &E);
    E -= 1; /* now 2^E <= a < 2^(E+1) */
    if (E < emin) E = emin; /* below the normal range the spacing stays 2^(emin - pbits) */
    /* a / spacing, where spacing = 2^(E - pbits); scaling by a power of two is exact, and
     * nearbyint rounds to the nearest integer, ties to even (default rounding mode). */
    double q = nearbyint(ldexp(a, pbits - E));
    if (q >= ldexp(1.0, pbits + 1)) { /* rounded up into the next binade */
        q = ldexp(q, -1);
        E += 1;
    }
    if (E > bias) return sign | (emax << pbits); /* beyond the largest finite value */
    uint32_t n = (uint32_t)q;
    if (n < (1u << pbits)) return sign | n; /* subnormal, E == emin */
    return sign | ((uint32_t)(E + bias) << pbits) | (n - (1u << pbits));
}

static double load_elem(const void* base, int64_t i, int dtype) {
    int ebits, pbits, bytes;
    format_of(dtype, &ebits, &pbits, &bytes);
    uint32_t bits;
    if (bytes == 4) {
        memcpy(&bits, (const unsigned char*)base + 4 * i, 4);
    } else {
        uint16_t h;
        memcpy(&h, (const unsigned char*)base + 2 * i, 2);
        bits = h;
    }
    return decode_bits(bits, ebits, pbits);
}

static void store_elem(void* base, int64_t i, double v, int dtype) {
    int ebits, pbits, bytes;
    format_of(dtype, &ebits, &pbits, &bytes);
    uint32_t bits = encode_bits(v, ebits, pbits);
    if (bytes == 4) {
        memcpy((unsigned char*)base + 4 * i, &bits, 4);
    } else {
        uint16_t h = (uint16_t)bits;
        memcpy((unsigned char*)base + 2 * i, &h, 2);
    }
}

double gtms_oracle_decode(uint32_t bits, int dtype) {
    int ebits, pbits, bytes;
    if (!format_of(dtype, &ebits, &pbits, &bytes)) return NAN;
    return decode_bits(bits, ebits, pbits);
}

uint32_t gtms_oracle_encode(double v, int dtype) {
    int ebits, pbits, bytes;
    if (!format_of(dtype, &ebits, &pbits, &bytes)) return 0;
    return encode_bits(v, ebits, pbits);
}

/* ------------------------------------------------------------------------------------
 * The operation.
 * ------------------------------------------------------------------------------------ */

/* Valid length of a batch: the raw value clamped to [0, S]. */
static int64_t valid_length(int32_t raw, int64_t S) {
    int64_t L = raw;
    if (L < 0) L = 0;
    if (L > S) L = S;
    return L;
}

/* The mask predicate of the operator-behaviour listing: an element is kept when neither
 * its row nor its column reaches the valid length and it lies on or below the diagonal. */
static int kept(int64_t row, int64_t col, int64_t L) {
    int invalid = row >= L || col >= L;
    return !invalid && row >= col;
}

/* One row of S elements at x (element type dtype), row index r, valid length L.
 * Writes S fp64 results to y. */
static void softmax_row(const void* x, int64_t r, int64_t L, int64_t S, double scale,
                        int dtype, double* y) {
    /* z_c = scale * x_c for the kept columns; mu = their maximum. */
    double mu = -INFINITY;
    int64_t nkept = 0;
    for (int64_t c = 0; c < S; ++c) {
        if (!kept(r, c, L)) continue;
        double z = scale * load_elem(x, c, dtype);
        if (z > mu) mu = z;
        ++nkept;
    }
    if (nkept == 0) { /* a padded row: every element is masked */
        for (int64_t c = 0; c < S; ++c) y[c] = 0.0;
        return;
    }
    /* denominator: sum over kept columns of exp(z_c - mu), in column order */
    double den = 0.0;
    for (int64_t c = 0; c < S; ++c) {
        if (!kept(r, c, L)) continue;
        den += exp(scale * load_elem(x, c, dtype) - mu);
    }
    for (int64_t c = 0; c < S; ++c) {
        if (kept(r, c, L))
            y[c] = exp(scale * load_elem(x, c, dtype) - mu) / den;
        else
            y[c] = 0.0;
    }
}

/* Checks shared by the entry points; on success *n_elem = B*M*S*S. */
static int check_shape(const void* a, const void* b, const int32_t* seq_lens, int64_t B,
                       int64_t M, int64_t S, int dtype, int64_t* n_elem) {
    int ebits, pbits, bytes;
    if (!format_of(dtype, &ebits, &pbits, &bytes)) return ERR_DTYPE;
    if (B < 0 || M < 0 || S < 0) return ERR_ARG;
    int64_t n = 1;
    if (__builtin_mul_overflow(n, B, &n) || __builtin_mul_overflow(n, M, &n) ||
        __builtin_mul_overflow(n, S, &n) || __builtin_mul_overflow(n, S, &n))
        return ERR_ARG;
    if (n > 0 && (!a || !b || !seq_lens)) return ERR_ARG;
    *n_elem = n;
    return OK;
}

int gtms_oracle_f64(const void* in, double* out, const int32_t* seq_lens, int64_t B,
                    int64_t M, int64_t S, float scale, int dtype) {
    int64_t n;
    int st = check_shape(in, out, seq_lens, B, M, S, dtype, &n);
    if (st != OK || n == 0) return st;
    int ebits, pbits, bytes;
    format_of(dtype, &ebits, &pbits, &bytes);
    for (int64_t b = 0; b < B; ++b) {
        int64_t L = valid_length(seq_lens[b], S);
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t r = 0; r < S; ++r) {
                int64_t off = ((b * M + m) * S + r) * S;
                softmax_row((const unsigned char*)in + off * bytes, r, L, S, (double)scale,
                            dtype, out + off);
            }
        }
    }
    return OK;
}

int gtms_oracle(const void* in, void* out, const int32_t* seq_lens, int64_t B, int64_t M,
                int64_t S, float scale, int dtype) {
    int64_t n;
    int st = check_shape(in, out, seq_lens, B, M, S, dtype, &n);
    if (st != OK || n == 0) return st;
    int ebits, pbits, bytes;
    format_of(dtype, &ebits, &pbits, &bytes);
    double* y = (double*)malloc((size_t)S * sizeof(double));
    if (!y) return ERR_ARG;
    for (int64_t b = 0; b < B; ++b) {
        int64_t L = valid_length(seq_lens[b], S);
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t r = 0; r < S; ++r) {
                int64_t off = ((b * M + m) * S + r) * S;
                softmax_row((const unsigned char*)in + off * bytes, r, L, S, (double)scale,
                            dtype, y);
                for (int64_t c = 0; c < S; ++c) store_elem(out, off + c, y[c], dtype);
            }
        }
    }
    free(y);
    return OK;
}

int gtms_oracle_rows_f64(const void* rows_in, double* rows_out, const int64_t* row,
                         const int32_t* seq_len, int64_t nrows, int64_t S, float scale,
                         int dtype) {
    int ebits, pbits, bytes;
    if (!format_of(dtype, &ebits, &pbits, &bytes)) return ERR_DTYPE;
    if (nrows < 0 || S < 0) return ERR_ARG;
    if (nrows == 0 || S == 0) return OK;
    if (!rows_in || !rows_out || !row || !seq_len) return ERR_ARG;
    for (int64_t i = 0; i < nrows; ++i) {
        if (row[i] < 0 || row[i] >= S) return ERR_ARG;
    }
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t L = valid_length(seq_len[i], S);
        softmax_row((const unsigned char*)rows_in + i * S * bytes, row[i], L, S,
                    (double)scale, dtype, rows_out + i * S);
    }
    return OK;
}

/* Backward. For one kept row, y = softmax(z) with z = scale * x, and the softmax
 * derivative dy_i/dz_j = y_i (delta_ij - y_j) (page "ops(8) self-attention CUDA (下)",
 * section 2.1, softmax derivative) gives, for an upstream gradient g,
 *   dx_j = scale * sum_i g_i y_i (delta_ij - y_j) = scale * y_j * (g_j - sum_i g_i y_i),
 * the sums running over the kept columns of the row. Masked elements and padded rows do
 * not reach the output, so their gradient is zero. */
static void backward_row(const void* y, const void* dy, int64_t off, int64_t r, int64_t L,
                         int64_t S, double scale, int dtype, double* dx) {
    double dot = 0.0;
    for (int64_t c = 0; c < S; ++c) {
        if (kept(r, c, L)) dot += load_elem(dy, off + c, dtype) * load_elem(y, off + c, dtype);
    }
    for (int64_t c = 0; c < S; ++c) {
        if (kept(r, c, L))
            dx[c] = scale * load_elem(y, off + c, dtype) * (load_elem(dy, off + c, dtype) - dot);
        else
            dx[c] = 0.0;
    }
}

int gtms_oracle_backward_f64(const void* y, const void* dy, double* dx,
                             const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                             float scale, int dtype) {
    int64_t n;
    int st = check_shape(y, dx, seq_lens, B, M, S, dtype, &n);
    if (st != OK || n == 0) return st;
    if (!dy) return ERR_ARG;
    for (int64_t b = 0; b < B; ++b) {
        int64_t L = valid_length(seq_lens[b], S);
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t r = 0; r < S; ++r) {
                int64_t off = ((b * M + m) * S + r) * S;
                backward_row(y, dy, off, r, L, S, (double)scale, dtype, dx + off);
            }
        }
    }
    return OK;
}

int gtms_oracle_backward_rows_f64(const void* y_rows, const void* dy_rows, double* dx_rows,
                                  const int64_t* row, const int32_t* seq_len, int64_t nrows,
                                  int64_t S, float scale, int dtype) {
    int ebits, pbits, bytes;
    if (!format_of(dtype, &ebits, &pbits, &bytes)) return ERR_DTYPE;
    if (nrows < 0 || S < 0) return ERR_ARG;
    if (nrows == 0 || S == 0) return OK;
    if (!y_rows || !dy_rows || !dx_rows || !row || !seq_len) return ERR_ARG;
    for (int64_t i = 0; i < nrows; ++i) {
        if (row[i] < 0 || row[i] >= S) return ERR_ARG;
    }
    for (int64_t i = 0; i < nrows; ++i) {
        backward_row(y_rows, dy_rows, i * S, row[i], valid_length(seq_len[i], S), S,
                     (double)scale, dtype, dx_rows + i * S);
    }
    return OK;
}

/* ------------------------------------------------------------------------------------
 * Mask variants. The page "优化ScaledMaskSoftmax算子" (ScaledMaskSoftmax article) applies a
 * softmax under a general mask: masked scores are set to minus infinity before the
 * exponentials (section 2.1), and a row whose every element is masked gives zeros
 * (section 4.1, the guard for an all-zero mask row). Section 6 builds such masks for a
 * local window (a lower-triangular band made with tril), for per-task masks broadcast
 * over the batch, and for per-sample valid lengths. Here the kept set of a row is given as
 * one flag per column, and the row's softmax runs over the flagged columns only.
 * ------------------------------------------------------------------------------------ */

/* Softmax of z_c = scale * x_c over the columns c with keep[c] != 0; other columns and rows
 * with no kept column give 0. */
static void softmax_kept_row(const void* x, const unsigned char* keep, int64_t S,
                             double scale, int dtype, double* y) {
    double mu = -INFINITY;
    int64_t nkept = 0;
    for (int64_t c = 0; c < S; ++c) {
        if (!keep[c]) continue;
        double z = scale * load_elem(x, c, dtype);
        if (z > mu) mu = z;
        ++nkept;
    }
    if (nkept == 0) {
        for (int64_t c = 0; c < S; ++c) y[c] = 0.0;
        return;
    }
    double den = 0.0;
    for (int64_t c = 0; c < S; ++c) {
        if (keep[c]) den += exp(scale * load_elem(x, c, dtype) - mu);
    }
    for (int64_t c = 0; c < S; ++c)
        y[c] = keep[c] ? exp(scale * load_elem(x, c, dtype) - mu) / den : 0.0;
}

/* Gradient of the same row with respect to x, given its output y and upstream gradient g
 * (the softmax derivative of the self-attention article, section 2.1, restricted to the
 * kept columns): dx_c = scale * y_c * (g_c - sum_k g_k y_k) on kept columns, else 0. */
static void backward_kept_row(const void* y, const void* g, const unsigned char* keep,
                              int64_t S, double scale, int dtype, double* dx) {
    double dot = 0.0;
    for (int64_t c = 0; c < S; ++c) {
        if (keep[c]) dot += load_elem(g, c, dtype) * load_elem(y, c, dtype);
    }
    for (int64_t c = 0; c < S; ++c)
        dx[c] = keep[c] ? scale * load_elem(y, c, dtype) * (load_elem(g, c, dtype) - dot) : 0.0;
}

/* Band predicate: element (r, c) of a batch with valid length L is kept when r < L, c < L
 * and lo <= c - r <= hi. lo <= -(S-1), hi = 0 is the grouped tril mask; hi = w alone is the
 * article's tril(w) window; lo = -(w-1), hi = 0 is a causal window of w columns. */
static int kept_band(int64_t r, int64_t c, int64_t L, int64_t lo, int64_t hi) {
    if (r >= L || c >= L) return 0;
    return c - r >= lo && c - r <= hi;
}

static int check_variant(const void* a, const void* b, int64_t B, int64_t M, int64_t S,
                         int dtype, int64_t* n_elem) {
    int ebits, pbits, bytes;
    if (!format_of(dtype, &ebits, &pbits, &bytes)) return ERR_DTYPE;
    if (B < 0 || M < 0 || S < 0) return ERR_ARG;
    int64_t n = 1;
    if (__builtin_mul_overflow(n, B, &n) || __builtin_mul_overflow(n, M, &n) ||
        __builtin_mul_overflow(n, S, &n) || __builtin_mul_overflow(n, S, &n))
        return ERR_ARG;
    if (n > 0 && (!a || !b)) return ERR_ARG;
    *n_elem = n;
    return OK;
}

/* The kept flags of row r of plane (b, m), for the band (mask == NULL) or an explicit mask
 * (element (b, m, r, c) at mask[b*sb + m*sm + r*sr + c], kept when non-zero). */
static void row_flags(const unsigned char* mask, int64_t sb, int64_t sm, int64_t sr,
                      int64_t lo, int64_t hi, int64_t b, int64_t m, int64_t r, int64_t L,
                      int64_t S, unsigned char* keep) {
    for (int64_t c = 0; c < S; ++c) {
        if (mask)
            keep[c] = r < L && c < L && mask[b * sb + m * sm + r * sr + c] != 0;
        else
            keep[c] = (unsigned char)kept_band(r, c, L, lo, hi);
    }
}

/* Shared loop of the variant entry points. y_or_x is the forward input (forward) or the
 * forward output (backward); g is the upstream gradient (backward) or NULL (forward). */
static int run_variant(const void* y_or_x, const void* g, double* out,
                       const unsigned char* mask, int64_t sb, int64_t sm, int64_t sr,
                       int64_t lo, int64_t hi, const int32_t* seq_lens, int64_t B,
                       int64_t M, int64_t S, float scale, int dtype) {
    int ebits, pbits, bytes;
    format_of(dtype, &ebits, &pbits, &bytes);
    unsigned char* keep = (unsigned char*)malloc((size_t)S);
    if (!keep) return ERR_ARG;
    for (int64_t b = 0; b < B; ++b) {
        int64_t L = seq_lens ? valid_length(seq_lens[b], S) : S;
        for (int64_t m = 0; m < M; ++m) {
            for (int64_t r = 0; r < S; ++r) {
                int64_t off = ((b * M + m) * S + r) * S;
                row_flags(mask, sb, sm, sr, lo, hi, b, m, r, L, S, keep);
                const unsigned char* row = (const unsigned char*)y_or_x + off * bytes;
                if (g)
                    backward_kept_row(row, (const unsigned char*)g + off * bytes, keep, S,
                                      (double)scale, dtype, out + off);
                else
                    softmax_kept_row(row, keep, S, (double)scale, dtype, out + off);
            }
        }
    }
    free(keep);
    return OK;
}

int gtms_oracle_band_f64(const void* in, double* out, const int32_t* seq_lens, int64_t B,
                         int64_t M, int64_t S, int64_t lo, int64_t hi, float scale,
                         int dtype) {
    int64_t n;
    int st = check_variant(in, out, B, M, S, dtype, &n);
    if (st != OK || n == 0) return st;
    return run_variant(in, NULL, out, NULL, 0, 0, 0, lo, hi, seq_lens, B, M, S, scale, dtype);
}

int gtms_oracle_band_backward_f64(const void* y, const void* dy, double* dx,
                                  const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                                  int64_t lo, int64_t hi, float scale, int dtype) {
    int64_t n;
    int st = check_variant(y, dx, B, M, S, dtype, &n);
    if (st != OK || n == 0) return st;
    if (!dy) return ERR_ARG;
    return run_variant(y, dy, dx, NULL, 0, 0, 0, lo, hi, seq_lens, B, M, S, scale, dtype);
}

int gtms_oracle_masked_f64(const void* in, double* out, const uint8_t* mask, int64_t mask_sb,
                           int64_t mask_sm, int64_t mask_sr, const int32_t* seq_lens,
                           int64_t B, int64_t M, int64_t S, float scale, int dtype) {
    int64_t n;
    int st = check_variant(in, out, B, M, S, dtype, &n);
    if (st != OK || n == 0) return st;
    if (!mask || mask_sb < 0 || mask_sm < 0 || mask_sr < 0) return ERR_ARG;
    return run_variant(in, NULL, out, mask, mask_sb, mask_sm, mask_sr, 0, 0, seq_lens, B, M,
                       S, scale, dtype);
}

int gtms_oracle_masked_backward_f64(const void* y, const void* dy, double* dx,
                                    const uint8_t* mask, int64_t mask_sb, int64_t mask_sm,
                                    int64_t mask_sr, const int32_t* seq_lens, int64_t B,
                                    int64_t M, int64_t S, float scale, int dtype) {
    int64_t n;
    int st = check_variant(y, dx, B, M, S, dtype, &n);
    if (st != OK || n == 0) return st;
    if (!dy || !mask || mask_sb < 0 || mask_sm < 0 || mask_sr < 0) return ERR_ARG;
    return run_variant(y, dy, dx, mask, mask_sb, mask_sm, mask_sr, 0, 0, seq_lens, B, M, S,
                       scale, dtype);
}

/* ------------------------------------------------------------------------------------
 * Attention with the grouped tril mask. The self-attention article ("ops(8) self-attention
 * CUDA", sections 1 and 2) computes attention as three steps: scores S = Q K^T, a softmax
 * of each score row, and O = P V. Here the softmax is this operation's: for batch b with
 * valid length L (clamped to [0, S]) and query row r < L, the row keeps the keys c <= r,
 * and
 *   O[r] = sum_{c <= r} p_c V[c],  p_c = exp(z_c - mu) / sum_{k <= r} exp(z_k - mu),
 *   z_c = scale * sum_d Q[r, d] K[c, d],
 * while a query row r >= L is all zeros (a padded row of the softmax gives P = 0).
 * Q, K, V and O are [B, M, S, D], row-major, in the element type; out receives fp64.
 * ------------------------------------------------------------------------------------ */
/* One query row r of a head: q, k and v point at the head's first element ([S, D]); o
 * receives D values; z is scratch for r + 1 scores. */
static void attention_row(const void* q, const void* k, const void* v, int64_t r, int64_t L,
                          int64_t D, double scale, int dtype, double* z, double* o) {
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    if (r >= L) return;
    /* scores of the kept keys c = 0..r and their maximum */
    double mu = -INFINITY;
    for (int64_t c = 0; c <= r; ++c) {
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d)
            dot += load_elem(q, r * D + d, dtype) * load_elem(k, c * D + d, dtype);
        z[c] = scale * dot;
        if (z[c] > mu) mu = z[c];
    }
    double den = 0.0;
    for (int64_t c = 0; c <= r; ++c) den += exp(z[c] - mu);
    for (int64_t c = 0; c <= r; ++c) {
        double p = exp(z[c] - mu) / den;
        for (int64_t d = 0; d < D; ++d) o[d] += p * load_elem(v, c * D + d, dtype);
    }
}

int gtms_oracle_attention_f64(const void* q, const void* k, const void* v, double* out,
                              const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                              int64_t D, float scale, int dtype) {
    int ebits, pbits, bytes;
    if (!format_of(dtype, &ebits, &pbits, &bytes)) return ERR_DTYPE;
    if (B < 0 || M < 0 || S < 0 || D < 0) return ERR_ARG;
    int64_t n = 1;
    if (__builtin_mul_overflow(n, B, &n) || __builtin_mul_overflow(n, M, &n) ||
        __builtin_mul_overflow(n, S, &n) || __builtin_mul_overflow(n, D, &n))
        return ERR_ARG;
    if (n == 0) return OK;
    if (!q || !k || !v || !out || !seq_lens) return ERR_ARG;
    double* z = (double*)malloc((size_t)S * sizeof(double));
    if (!z) return ERR_ARG;
    for (int64_t b = 0; b < B; ++b) {
        int64_t L = valid_length(seq_lens[b], S);
        for (int64_t m = 0; m < M; ++m) {
            int64_t head = (b * M + m) * S * D;  /* first element of this head's [S, D] */
            for (int64_t r = 0; r < S; ++r)
                attention_row((const unsigned char*)q + head * bytes,
                              (const unsigned char*)k + head * bytes,
                              (const unsigned char*)v + head * bytes, r, L, D, (double)scale,
                              dtype, z, out + head + r * D);
        }
    }
    free(z);
    return OK;
}

int gtms_oracle_attention_row_f64(const void* q, const void* k, const void* v, double* out,
                                  int64_t r, int32_t seq_len, int64_t S, int64_t D,
                                  float scale, int dtype) {
    int ebits, pbits, bytes;
    if (!format_of(dtype, &ebits, &pbits, &bytes)) return ERR_DTYPE;
    if (S < 0 || D < 0 || r < 0 || r >= S) return ERR_ARG;
    if (!q || !k || !v || !out) return ERR_ARG;
    double* z = (double*)malloc((size_t)(r + 1) * sizeof(double));
    if (!z) return ERR_ARG;
    attention_row(q, k, v, r, valid_length(seq_len, S), D, (double)scale, dtype, z, out);
    free(z);
    return OK;
}
