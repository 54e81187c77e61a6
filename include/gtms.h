/*
 * gtms: grouped tril mask softmax on AMD Instinct MI355X (gfx950, CDNA4).
 *
 * The operation (page "Fused grouped tril mask softmax", github aoxy/Attention-Mask-
 * Optimization README, operator-behaviour section and the masks printed after it):
 * X holds attention scores of shape [B, M, S, S], row-major and contiguous. Every plane of
 * batch b shares one valid length L_b = clamp(seq_lens[b], 0, S). For row r < L_b the
 * output row is softmax(scale * X[b, m, r, 0..r]) in columns 0..r and +0.0 in columns
 * r+1..S-1; every row r >= L_b is written as +0.0. The mask is computed from (r, c, L_b)
 * and never loaded, and masked scores do not influence the result. The scale multiplies
 * the scores before the softmax (page "优化ScaledMaskSoftmax算子", sections 2.1 and 4.1).
 *
 * Element types: binary32, binary16 and bfloat16 in memory; arithmetic in fp32 on the GPU
 * (the mixed-precision scheme of the ScaledMaskSoftmax article, section 2.1). Results are
 * rounded to nearest, ties to even, into the element type.
 *
 * Conventions of every entry point:
 *   - all pointers are device pointers, owned by the caller; the library allocates no
 *     memory and keeps no state between calls, so calls are re-entrant;
 *   - work is queued on `stream` (a hipStream_t; NULL is the null stream) and the call
 *     returns without waiting; the caller synchronises before reading results;
 *   - B * M * S == 0 is a valid no-op;
 *   - seq_lens values outside [0, S] are clamped on the device (they live in device
 *     memory, so the host never inspects them);
 *   - errors are returned as a gtms_status; nothing aborts and no exception crosses the
 *     ABI. A failed call queues no work.
 */
#ifndef GTMS_H
#define GTMS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type codes. */
enum gtms_dtype { GTMS_F32 = 0, GTMS_F16 = 1, GTMS_BF16 = 2 };

/* Status codes returned by every entry point. */
enum gtms_status {
    GTMS_OK = 0,
    GTMS_ERR_INVALID_ARG = 1, /* negative size or mask stride, null pointer, B*M*S*S
                                 overflows int64, S above GTMS_MAX_S, or in/out partially
                                 overlapping */
    GTMS_ERR_DTYPE = 2,       /* unknown element type code */
    GTMS_ERR_ALIGN = 3,       /* a pointer not aligned to its element size */
    GTMS_ERR_HIP = 4,         /* the HIP runtime refused the launch */
    GTMS_ERR_PATH = 5         /* gtms_forward_ex: unknown path, or a path that cannot
                                 serve this shape and alignment */
};

/* Largest supported row length. */
#define GTMS_MAX_S (1 << 24)

/*
 * Forward: out = grouped tril mask softmax of in.
 *   in, out   [B, M, S, S] elements of `dtype`, contiguous row-major. in == out (in place,
 *             as the README's listing overwrites its scores) is allowed; any other overlap
 *             is rejected with GTMS_ERR_INVALID_ARG.
 *   seq_lens  B int32 valid lengths.
 *   scale     multiplies the scores before the softmax; |scale * x * log2(e)| must stay
 *             inside the fp32 range for the kept scores.
 * Rows whose kept scores hold NaN or infinity produce NaN in their kept columns; their
 * masked columns are still +0.0.
 */
int gtms_forward(const void* in, void* out, const int32_t* seq_lens, int64_t B, int64_t M,
                 int64_t S, float scale, int dtype, void* stream);

/* Kernel choice for gtms_forward_ex. AUTO is what gtms_forward uses. A lane holds up to
 * 16 vectors: 16-byte vectors when the row's byte length is a multiple of 16 and both
 * tensors are 16-byte aligned, single elements otherwise. */
enum gtms_path {
    GTMS_PATH_AUTO = 0,
    GTMS_PATH_WAVE = 1,   /* one 64-lane wavefront per row, the row held in registers:
                             rows up to 1024 vectors (4096 binary32 / 8192 16-bit
                             elements on aligned rows) */
    GTMS_PATH_BLOCK = 2,  /* one workgroup of 2-16 wavefronts per row, per-wave (max, sum)
                             partials merged through LDS: rows up to 16384 vectors. The
                             backward of the computed masks on 16-byte vectors holds rows
                             past 8192 vectors as 8192 in registers and up to 5056 more of
                             y and dy in LDS (16-bit rows up to 105984 elements, binary32
                             up to 52992); longer rows there use 16 vectors per lane in
                             registers */
    GTMS_PATH_STREAM = 3  /* one workgroup per row, two passes over the row: online
                             (max, sum), then normalise (any row length) */
};

/* Option bits for gtms_forward_ex (0 = the defaults gtms_forward uses). */
enum gtms_flags {
    GTMS_FLAG_PAIR_ROWS = 1u << 0,  /* one work unit = rows r and S-1-r (equal prefix work per
                                       unit; slower on MI355X, where adjacent rows written
                                       together keep HBM accesses local) */
    GTMS_FLAG_PLAIN_ORDER = 1u << 1 /* hand work to the XCDs in the hardware's round-robin
                                       block order. By default the blocks are renumbered so
                                       that each XCD works through chunks of 16 consecutive
                                       blocks, which keeps each XCD's accesses in one stretch
                                       of memory; that measured 4-10% faster on MI355X */
};

/*
 * Forward with an explicit kernel choice and options. For one path every flag setting
 * gives the same bits; different paths reduce in different orders, so they agree with each
 * other only to within rounding. A path that cannot serve the shape (row too long for its
 * registers) returns GTMS_ERR_PATH. Meant for tests and tuning.
 */
int gtms_forward_ex(const void* in, void* out, const int32_t* seq_lens, int64_t B,
                    int64_t M, int64_t S, float scale, int dtype, int path, unsigned flags,
                    void* stream);

/*
 * Backward: dx = gradient of the forward with respect to its input, given the forward
 * output y and the upstream gradient dy. For a kept element (r < L_b, c <= r)
 *   dx[c] = scale * y[c] * (dy[c] - sum_{k <= r} dy[k] * y[k]),
 * from the softmax derivative dy_i/dz_j = y_i (delta_ij - y_j) (page "ops(8) self-attention
 * CUDA (下)", section 2.1); every other element is +0.0.
 *   y, dy, dx [B, M, S, S] elements of `dtype`; dx may be dy itself (in place) but must
 *             not overlap y, nor overlap dy partially (GTMS_ERR_INVALID_ARG).
 * Arithmetic fp32, results rounded to nearest-even. Other conventions as for gtms_forward.
 */
int gtms_backward(const void* y, const void* dy, void* dx, const int32_t* seq_lens,
                  int64_t B, int64_t M, int64_t S, float scale, int dtype, void* stream);

/* Backward with an explicit kernel choice and options (as gtms_forward_ex). */
int gtms_backward_ex(const void* y, const void* dy, void* dx, const int32_t* seq_lens,
                     int64_t B, int64_t M, int64_t S, float scale, int dtype, int path,
                     unsigned flags, void* stream);

/*
 * Mask variants (page "优化ScaledMaskSoftmax算子", the ScaledMaskSoftmax article): masked
 * scores count as minus infinity before the softmax (section 2.1), and a row with no kept
 * element is written as +0.0 (section 4.1, the guard for an all-masked row). Section 6 of
 * the article builds such masks for a local window (with tril), per task (one mask
 * broadcast over the batch) and per sample (positions below each sample's length); the
 * two variants below cover those cases.
 *
 * Common to both: seq_lens may be NULL, which means every valid length is S; otherwise an
 * element (r, c) of batch b can only be kept when r < L_b and c < L_b. Layout, dtype,
 * in-place rules, streams and errors are those of gtms_forward / gtms_backward. Each row's
 * softmax runs over its kept elements; every other element is +0.0.
 */

/*
 * Band: element (r, c) is kept when lo <= c - r <= hi. The mask is computed, never loaded.
 *   lo <= -(S-1), hi = 0      the grouped tril mask of gtms_forward (same results)
 *   lo <= -(S-1), hi = w      the article's window mask tril(w)
 *   lo = -(w-1), hi = 0       a causal sliding window of w columns
 *   lo > hi                   every row is +0.0
 * Any int64 values are accepted (c - r always lies in [-(S-1), S-1]).
 */
int gtms_forward_band(const void* in, void* out, const int32_t* seq_lens, int64_t B,
                      int64_t M, int64_t S, int64_t lo, int64_t hi, float scale, int dtype,
                      void* stream);

/* Band forward with an explicit kernel choice and options (as gtms_forward_ex). */
int gtms_forward_band_ex(const void* in, void* out, const int32_t* seq_lens, int64_t B,
                         int64_t M, int64_t S, int64_t lo, int64_t hi, float scale, int dtype,
                         int path, unsigned flags, void* stream);

/*
 * Explicit mask: element (b, m, r, c) is kept when the byte
 *   mask[b * mask_stride_b + m * mask_stride_m + r * mask_stride_r + c]
 * is non-zero (the reading of the article's mask where 1 marks a position to attend, as
 * its section-6 examples build them). Strides are in bytes and must be >= 0; a stride of
 * 0 broadcasts that dimension, so one [S, S] mask (strides 0, 0, S), per-batch or
 * per-head masks, and per-sample key masks [B, 1, 1, S] (strides S, 0, 0) all fit. The
 * column stride is 1. The caller guarantees that the S bytes of every mask row addressed
 * for a row r < L_b lie in device memory (kernels read whole vectors, so columns up to
 * the next multiple of 16 / element size past L_b - 1 may be read); the library cannot
 * check the mask's extent. The mask may alias nothing that the call writes. With 16-byte vectors the mask's base
 * address and strides must be multiples of 16 / element size (4 for binary32, 8 for
 * 16-bit types); otherwise the call takes the element-wise path, which is slower but
 * accepts any layout.
 */
int gtms_forward_masked(const void* in, void* out, const uint8_t* mask, int64_t mask_stride_b,
                        int64_t mask_stride_m, int64_t mask_stride_r, const int32_t* seq_lens,
                        int64_t B, int64_t M, int64_t S, float scale, int dtype, void* stream);

/* Explicit-mask forward with an explicit kernel choice and options. */
int gtms_forward_masked_ex(const void* in, void* out, const uint8_t* mask,
                           int64_t mask_stride_b, int64_t mask_stride_m, int64_t mask_stride_r,
                           const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                           float scale, int dtype, int path, unsigned flags, void* stream);

/*
 * Backward of the two variants: dx[c] = scale * y[c] * (dy[c] - sum over kept k of
 * dy[k] * y[k]) on kept elements, +0.0 elsewhere (the derivative used by gtms_backward,
 * over the variant's kept set). Arguments as gtms_backward_ex plus the variant's mask.
 */
int gtms_backward_band(const void* y, const void* dy, void* dx, const int32_t* seq_lens,
                       int64_t B, int64_t M, int64_t S, int64_t lo, int64_t hi, float scale,
                       int dtype, int path, unsigned flags, void* stream);
int gtms_backward_masked(const void* y, const void* dy, void* dx, const uint8_t* mask,
                         int64_t mask_stride_b, int64_t mask_stride_m, int64_t mask_stride_r,
                         const int32_t* seq_lens, int64_t B, int64_t M, int64_t S, float scale,
                         int dtype, int path, unsigned flags, void* stream);

/*
 * Attention with the grouped tril mask, fused (the self-attention article, "ops(8)
 * self-attention CUDA": scores, row softmax, weighted sum of values; here the softmax is
 * the grouped tril mask softmax of gtms_forward):
 *   for query row r < L_b:  out[r] = sum_{c <= r} softmax_c(scale * q[r] . k[c]) v[c]
 *   for query row r >= L_b: out[r] = 0
 * q, k, v, out  [B, M, S, D] elements of `dtype`, row-major, contiguous: M heads per batch
 *               entry, S positions, head size D. out may overlap none of q, k, v.
 * seq_lens      B int32 valid lengths (clamped to [0, S] on the device).
 * dtype         GTMS_F16 or GTMS_BF16 (GTMS_ERR_DTYPE otherwise); the scores, the softmax
 *               and the sums are fp32; the probabilities are rounded to `dtype` before the
 *               product with v (matrix-core operands); out is rounded to nearest-even.
 * D             64 or 128 (GTMS_ERR_PATH otherwise).
 * scale         any finite value; 0 and -0 give the mean of v over the keys c <= r.
 * All pointers 16-byte aligned (GTMS_ERR_ALIGN). One head (S * D elements) must be below
 * 2^30 elements. The S x S scores are never written to memory.
 * Values at positions >= L_b of q, k and v are never read into a result. Below L_b, v
 * must be finite: the products of up to 127 later keys of the same 128-row query tile
 * are formed with probability 0, so a NaN or infinity in v[c] can reach rows r < c of
 * that tile (0 * inf is NaN). Non-finite q or k below L_b affect only the rows that
 * attend to them.
 */
int gtms_attention_forward(const void* q, const void* k, const void* v, void* out,
                           const int32_t* seq_lens, int64_t B, int64_t M, int64_t S, int64_t D,
                           float scale, int dtype, void* stream);

/* Work split of the fused attention for gtms_attention_forward_ex. Each workgroup computes
 * one 128-row query tile of one head; at head size 64 it can instead hold two groups of four
 * wavefronts that take the first and second half of the tile's key blocks, each with its own
 * running (max, sum) and accumulators, merged at the end as the split-KV reduction of
 * flash_decoding.py does (the page "flash_decoding.py", _flash_decoding_fwd_reduce_kernel):
 * m = max of the parts' maxima, l = sum of l_i 2^(m_i - m), out = sum of out_i 2^(m_i - m).
 * That halves the longest chain of key blocks, which sets the launch's length when a grid
 * has few tiles per compute unit. AUTO (what gtms_attention_forward uses) takes the split
 * at head size 64 when S >= 2048 and the grid has at most 3 (head, tile) pairs per compute
 * unit of the device. The two choices reduce in different orders, so they agree to within
 * rounding. */
enum gtms_attn_split {
    GTMS_ATTN_SPLIT_AUTO = 0,
    GTMS_ATTN_SPLIT_OFF = 1,
    GTMS_ATTN_SPLIT_ON = 2  /* head size 64 only; at 128 the choice is ignored */
};

/* gtms_attention_forward with an explicit work split (a GTMS_ATTN_SPLIT_* value; others give
 * GTMS_ERR_PATH). Meant for tests and tuning. */
int gtms_attention_forward_ex(const void* q, const void* k, const void* v, void* out,
                              const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                              int64_t D, float scale, int dtype, int split, void* stream);

/* A static, human-readable description of a status code. */
const char* gtms_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch. */
int gtms_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GTMS_H */
