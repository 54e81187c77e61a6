// C ABI of the gtms library: argument checks, kernel choice and launches.
// Declarations and the contract of every entry point are in include/gtms.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "gtms.h"
#include "launch.h"

namespace gtms {
namespace {

// Each XCD takes chunks of 2^4 consecutive blocks (unless GTMS_FLAG_PLAIN_ORDER). Measured on
// MI355X over chunk sizes of 1 to 4096 blocks: 16 was fastest on every workload and path
// (binary32 rows of 1000 elements four to a block, 16-bit rows of 4096 and 8192 elements one
// to a block), 4-10% above the plain round-robin order.
constexpr uint32_t kXcdChunkLog2 = 4;
// Rows per block of the unit order of shared explicit masks (F_ACROSS): 2^6 (2^8 measured
// 1.5% slower forward on bf16 rows of 65536 and within noise backward).
constexpr uint32_t kAcrossRowsLog2 = 6;

int esize_of(int dtype) { return dtype == GTMS_F32 ? 4 : 2; }

int64_t pow2_at_least(int64_t n) {
    int64_t p = 1;
    while (p < n) p <<= 1;
    return p;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shared argument checks; on success fills the byte count of one [B, M, S, S] tensor.
int check_common(const void* a, const void* b, const int32_t* seq_lens, bool lens_optional,
                 int64_t B, int64_t M, int64_t S, int dtype, int64_t* bytes, bool* empty) {
    if (dtype != GTMS_F32 && dtype != GTMS_F16 && dtype != GTMS_BF16) return GTMS_ERR_DTYPE;
    if (B < 0 || M < 0 || S < 0 || S > GTMS_MAX_S || M > INT32_MAX) return GTMS_ERR_INVALID_ARG;
    int64_t n = esize_of(dtype);
    if (__builtin_mul_overflow(n, B, &n) || __builtin_mul_overflow(n, M, &n) ||
        __builtin_mul_overflow(n, S, &n) || __builtin_mul_overflow(n, S, &n))
        return GTMS_ERR_INVALID_ARG;
    *bytes = n;
    *empty = (n == 0);
    if (*empty) return GTMS_OK;
    if (!a || !b || (!seq_lens && !lens_optional)) return GTMS_ERR_INVALID_ARG;
    const uintptr_t es = (uintptr_t)esize_of(dtype);
    if ((uintptr_t)a % es || (uintptr_t)b % es || (uintptr_t)seq_lens % 4) return GTMS_ERR_ALIGN;
    return GTMS_OK;
}

bool overlap_partial(const void* a, const void* b, int64_t bytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    if (x == y) return false;
    return x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes;
}

// Leading slots a row may take over from the previous row under line ownership: rows
// start at base + k * row_bytes, so on a 128-byte aligned tensor the previous row's tail
// zone is a multiple of gcd(row_bytes, 128) bytes below 128.
int64_t line_slack(bool lines, int64_t row_bytes, const void* out) {
    if (!lines) return 0;
    if ((uintptr_t)out % 128) return 7;
    int64_t g = 128, b = row_bytes % 128;
    while (b) {
        const int64_t t = g % b;
        g = b;
        b = t;
    }
    return (128 - g) / 16;
}

// Kernel choice. A lane holds NV vectors (16 bytes each on rows whose byte length is a
// multiple of 16, else one element); a row takes 64 * W * NV slots: the vectors it may span,
// counting those it may write for its predecessor (line_slack), or for a narrow band only its
// interval's vectors (the rest are plain zero stores).
//   auto:   rows up to 256 slots -> one wavefront per row (NV <= 4); longer rows -> W
//           wavefronts per row with NV = 4 (the stores of each instruction then cover
//           W KB of the row); W = 16 and NV up to auto_max_nv beyond that; then, where
//           stash_cap > 0 (the backward of the computed masks on 16-byte vectors), W = 16
//           with 8 vectors per lane in registers and up to stash_cap more per row in LDS;
//           the stream path last.
//   forced: the named path if it can hold the row (the block path at 16 vectors per lane
//           takes the LDS stash when stash_cap > 0 and the row fits it).
int make_plan(int64_t slots, bool wide, int path, int64_t auto_max_nv, int64_t stash_cap,
              Plan* p) {
    p->wide = wide;
    p->stash = false;
    const int64_t stash_slots = int64_t(kWave) * kMaxW * kAutoMaxNV + stash_cap;
    if (path == GTMS_PATH_AUTO) {
        if (slots <= kWave * kAutoNV) path = GTMS_PATH_WAVE;
        else if (slots <= int64_t(kWave) * kMaxW * auto_max_nv) path = GTMS_PATH_BLOCK;
        else if (stash_cap > 0 && slots <= stash_slots) path = GTMS_PATH_BLOCK;
        else path = GTMS_PATH_STREAM;
    }
    p->path = path;
    switch (path) {
        case GTMS_PATH_WAVE:
            if (slots > int64_t(kWave) * kMaxNV) return GTMS_ERR_PATH;
            p->nv = (int)pow2_at_least(cdiv(slots, kWave));
            p->w = 1;
            return GTMS_OK;
        case GTMS_PATH_BLOCK: {
            int64_t w = pow2_at_least(cdiv(slots, int64_t(kWave) * kAutoNV));
            if (w < 2) w = 2;
            if (w > kMaxW) w = kMaxW;
            const int64_t nv = pow2_at_least(cdiv(slots, int64_t(kWave) * w));
            if (nv > kMaxNV) return GTMS_ERR_PATH;
            p->w = (int)w;
            p->nv = (int)nv;
            p->stash = stash_cap > 0 && nv > kAutoMaxNV && w == kMaxW && slots <= stash_slots;
            return GTMS_OK;
        }
        case GTMS_PATH_STREAM:
            p->nv = 0;
            p->w = kStreamW;
            return GTMS_OK;
        default:
            return GTMS_ERR_PATH;
    }
}

// Which elements a call keeps (beyond r < L, c < L): MK_TRIL c <= r; MK_BAND
// lo <= c - r <= hi; MK_MASK a non-zero byte of `mask` (byte strides sb, sm, sr).
struct MaskSpec {
    int kind = MK_TRIL;
    int64_t lo = 0, hi = 0;
    const uint8_t* mask = nullptr;
    int64_t sb = 0, sm = 0, sr = 0;
};

// Shared body of the forward (x -> out) and backward (x = y, g = dy -> out = dx) calls.
template <int OP>
int run_impl(const void* x, const void* g, void* out, const int32_t* seq_lens, int64_t B,
             int64_t M, int64_t S, float scale, int dtype, int path, unsigned flags,
             void* stream, const MaskSpec& mk = MaskSpec()) {
    int64_t bytes;
    bool empty;
    int st = check_common(x, out, seq_lens, mk.kind != MK_TRIL, B, M, S, dtype, &bytes, &empty);
    if (st != GTMS_OK) return st;
    if (path < GTMS_PATH_AUTO || path > GTMS_PATH_STREAM) return GTMS_ERR_PATH;
    if (mk.kind == MK_MASK && (mk.sb < 0 || mk.sm < 0 || mk.sr < 0)) return GTMS_ERR_INVALID_ARG;
    if (empty) return GTMS_OK;
    if (mk.kind == MK_MASK && !mk.mask) return GTMS_ERR_INVALID_ARG;
    if (OP == OP_BWD) {
        if (!g) return GTMS_ERR_INVALID_ARG;
        if ((uintptr_t)g % esize_of(dtype)) return GTMS_ERR_ALIGN;
        // dx may replace dy, but must not touch y or overlap dy partially
        if (overlap_partial(g, out, bytes) || overlap_partial(x, out, bytes) || x == out)
            return GTMS_ERR_INVALID_ARG;
    } else if (overlap_partial(x, out, bytes)) {
        return GTMS_ERR_INVALID_ARG;
    }

    const int vec = 16 / esize_of(dtype);
    // 16-byte vectors need aligned rows of scores and, for an explicit mask, mask rows
    // whose VEC bytes per vector sit at multiples of VEC
    const bool mask_wide = mk.kind != MK_MASK ||
                           ((uintptr_t)mk.mask % vec == 0 && mk.sb % vec == 0 &&
                            mk.sm % vec == 0 && mk.sr % vec == 0);
    const bool wide = S % vec == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)out % 16 == 0 &&
                      (OP == OP_FWD || (uintptr_t)g % 16 == 0) && mask_wide;
    // whole-line writes at row boundaries (wave and block paths, rows of 16-byte vectors)
    const int64_t row_bytes = S * esize_of(dtype);
    const bool lines = wide && row_bytes >= 128 && path != GTMS_PATH_STREAM;
    Plan plan;
    // the block path's widest automatic layout: 16 vectors per lane for the forward of the
    // computed masks (their row parts keep raw vectors only, see RowPart), 8 otherwise
    const int64_t auto_max_nv =
        OP == OP_FWD && mk.kind != MK_MASK && wide ? kAutoMaxNVRaw : kAutoMaxNV;
    // A band narrower than the row holds only its interval in registers (F_IVREL), widened to
    // whole 128-byte lines: at most ceil(width / VEC) + 1 vectors (the interval need not start
    // on a vector boundary) plus up to a line less one vector at each end.
    const int64_t vecn = wide ? vec : 1;
    const int64_t per_line = 128 / (wide ? 16 : esize_of(dtype));
    const int64_t band_width = mk.kind == MK_BAND
        ? (mk.hi < S - 1 ? mk.hi : S - 1) - (mk.lo > -(S - 1) ? mk.lo : -(S - 1)) + 1
        : S;
    const int64_t iv_slots =
        (band_width <= 0 ? 1 : cdiv(band_width, vecn) + (vecn > 1)) + 2 * (per_line - 1);
    const int64_t row_slots = cdiv(S, vecn) + line_slack(lines, row_bytes, out);
    const bool ivrel = mk.kind == MK_BAND && band_width < S && iv_slots < row_slots;
    const int64_t slots = ivrel ? iv_slots : row_slots;
    // the backward's LDS stash holds 16-byte vectors of y and g, for the computed masks
    const int64_t stash_cap = OP == OP_BWD && mk.kind != MK_MASK && wide ? kStashVecs : 0;
    st = make_plan(slots, wide, path, auto_max_nv, stash_cap, &plan);
    if (st != GTMS_OK) return st;

    FwdArgs a;
    a.x = x;
    a.y = out;
    a.g = g;
    a.seq_lens = seq_lens;
    a.M = (uint32_t)M;
    a.S = (int)S;
    a.row_bytes = (int)row_bytes;
    a.flags = 0;
    if (flags & GTMS_FLAG_PAIR_ROWS) a.flags |= F_PAIR;
    if (!(flags & GTMS_FLAG_PLAIN_ORDER)) a.flags |= F_XCD;
    a.xcd_shift = kXcdChunkLog2;
    if (lines && plan.path != GTMS_PATH_STREAM) a.flags |= F_LINES;
    if (ivrel) a.flags |= F_IVREL;
    // An explicit mask whose rows the heads of a batch share (head stride 0), with two or
    // more planes on one mask row, on rows of 64 KB or more: units run in blocks of 2^6 rows
    // taken plane after plane (in the kernels of long rows, which are the ones such rows
    // get), so that each block of mask rows is fetched into an XCD's L2 about once for all
    // the planes instead of once per plane. Measured on MI355X with a
    // [1, 1, S, S] mask: bf16 rows of 65536 (2 x 2 planes) +7% forward and about +3%
    // backward; on rows of 2-16 KB (1000 f32, 4096 f16, 8192 bf16) the same order lost 3-12%
    // (their thousands of rows in flight then spread over several planes' blocks).
    if (mk.kind == MK_MASK && mk.sm == 0 && (M > 1 || (mk.sb == 0 && B > 1)) &&
        row_bytes >= 65536)
        a.flags |= F_ACROSS;
    a.across_shift = kAcrossRowsLog2;
    a.units_per_plane = (a.flags & F_PAIR) ? (uint32_t)((S + 1) / 2) : (uint32_t)S;
    const int64_t units = B * M * (int64_t)a.units_per_plane;
    if (units > (int64_t)UINT32_MAX || B * M > (int64_t)UINT32_MAX) return GTMS_ERR_INVALID_ARG;
    a.n_units = (uint32_t)units;
    a.n_planes = (uint32_t)(B * M);
    // forward: scale * log2(e), so that exp is 2^x; backward: the scale itself
    a.k = OP == OP_FWD ? (float)((double)scale * 1.4426950408889634074) : scale;
    // c - r lies in [-(S-1), S-1], so clamping the band to [-S, S] changes nothing
    a.lo = (int)(mk.lo < -S ? -S : (mk.lo > S ? S : mk.lo));
    a.hi = (int)(mk.hi < -S ? -S : (mk.hi > S ? S : mk.hi));
    a.mask = mk.mask;
    a.mask_sb = mk.sb;
    a.mask_sm = mk.sm;
    a.mask_sr = mk.sr;

    hipStream_t hs = (hipStream_t)stream;
    hipError_t e;
    switch (mk.kind) {
        case MK_TRIL: e = launch_kind<OP, MK_TRIL>(dtype, plan, a, hs); break;
        case MK_BAND: e = launch_kind<OP, MK_BAND>(dtype, plan, a, hs); break;
        default: e = launch_kind<OP, MK_MASK>(dtype, plan, a, hs); break;
    }
    return e == hipSuccess ? GTMS_OK : GTMS_ERR_HIP;
}

int attention_impl(const void* q, const void* k, const void* v, void* out,
                   const int32_t* seq_lens, int64_t B, int64_t M, int64_t S, int64_t D,
                   float scale, int dtype, int split, void* stream) {
    if (dtype != GTMS_F16 && dtype != GTMS_BF16) return GTMS_ERR_DTYPE;
    if (split < GTMS_ATTN_SPLIT_AUTO || split > GTMS_ATTN_SPLIT_ON) return GTMS_ERR_PATH;
    if (B < 0 || M < 0 || S < 0 || D < 0 || S > GTMS_MAX_S || M > INT32_MAX)
        return GTMS_ERR_INVALID_ARG;
    int64_t planes = 0, bytes = 0;
    if (__builtin_mul_overflow(B, M, &planes) || __builtin_mul_overflow(planes, S * D * 2, &bytes))
        return GTMS_ERR_INVALID_ARG;
    // one head's byte offsets, up to the last query tile's end, stay below 2^31
    if ((S + kAttnRows) * D * 2 >= (int64_t(1) << 31)) return GTMS_ERR_INVALID_ARG;
    if (bytes == 0) return GTMS_OK;
    if (D != 64 && D != 128) return GTMS_ERR_PATH;
    if (!q || !k || !v || !out || !seq_lens) return GTMS_ERR_INVALID_ARG;
    if ((uintptr_t)q % 16 || (uintptr_t)k % 16 || (uintptr_t)v % 16 || (uintptr_t)out % 16 ||
        (uintptr_t)seq_lens % 4)
        return GTMS_ERR_ALIGN;
    // the output may overlap no input: blocks read keys and values of rows other blocks write
    for (const void* in : {q, k, v}) {
        const uintptr_t x = (uintptr_t)in, y = (uintptr_t)out;
        if (x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes) return GTMS_ERR_INVALID_ARG;
    }
    const int64_t tiles = (S + kAttnRows - 1) / kAttnRows;
    if (planes > (int64_t)UINT32_MAX || planes * tiles > (int64_t)INT32_MAX)
        return GTMS_ERR_INVALID_ARG;
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = out;
    a.seq_lens = seq_lens;
    a.n_planes = (uint32_t)planes;
    a.M = (uint32_t)M;
    a.S = (int)S;
    a.n_tiles = (int)tiles;
    a.k2 = (float)((double)scale * 1.4426950408889634074);
    const hipError_t e = launch_attention(dtype, (int)D, a, split, (hipStream_t)stream);
    return e == hipSuccess ? GTMS_OK : GTMS_ERR_HIP;
}

MaskSpec band(int64_t lo, int64_t hi) {
    MaskSpec m;
    m.kind = MK_BAND;
    m.lo = lo;
    m.hi = hi;
    return m;
}

MaskSpec explicit_mask(const uint8_t* mask, int64_t sb, int64_t sm, int64_t sr) {
    MaskSpec m;
    m.kind = MK_MASK;
    m.mask = mask;
    m.sb = sb;
    m.sm = sm;
    m.sr = sr;
    return m;
}

}  // namespace
}  // namespace gtms

extern "C" {

int gtms_forward(const void* in, void* out, const int32_t* seq_lens, int64_t B, int64_t M,
                 int64_t S, float scale, int dtype, void* stream) {
    return gtms::run_impl<gtms::OP_FWD>(in, nullptr, out, seq_lens, B, M, S, scale, dtype,
                                        GTMS_PATH_AUTO, 0u, stream);
}

int gtms_forward_ex(const void* in, void* out, const int32_t* seq_lens, int64_t B,
                    int64_t M, int64_t S, float scale, int dtype, int path, unsigned flags,
                    void* stream) {
    return gtms::run_impl<gtms::OP_FWD>(in, nullptr, out, seq_lens, B, M, S, scale, dtype, path,
                                        flags, stream);
}

int gtms_backward(const void* y, const void* dy, void* dx, const int32_t* seq_lens, int64_t B,
                  int64_t M, int64_t S, float scale, int dtype, void* stream) {
    return gtms::run_impl<gtms::OP_BWD>(y, dy, dx, seq_lens, B, M, S, scale, dtype,
                                        GTMS_PATH_AUTO, 0u, stream);
}

int gtms_backward_ex(const void* y, const void* dy, void* dx, const int32_t* seq_lens,
                     int64_t B, int64_t M, int64_t S, float scale, int dtype, int path,
                     unsigned flags, void* stream) {
    return gtms::run_impl<gtms::OP_BWD>(y, dy, dx, seq_lens, B, M, S, scale, dtype, path, flags,
                                        stream);
}

int gtms_forward_band(const void* in, void* out, const int32_t* seq_lens, int64_t B,
                      int64_t M, int64_t S, int64_t lo, int64_t hi, float scale, int dtype,
                      void* stream) {
    return gtms::run_impl<gtms::OP_FWD>(in, nullptr, out, seq_lens, B, M, S, scale, dtype,
                                        GTMS_PATH_AUTO, 0u, stream, gtms::band(lo, hi));
}

int gtms_forward_band_ex(const void* in, void* out, const int32_t* seq_lens, int64_t B,
                         int64_t M, int64_t S, int64_t lo, int64_t hi, float scale, int dtype,
                         int path, unsigned flags, void* stream) {
    return gtms::run_impl<gtms::OP_FWD>(in, nullptr, out, seq_lens, B, M, S, scale, dtype, path,
                                        flags, stream, gtms::band(lo, hi));
}

int gtms_forward_masked(const void* in, void* out, const uint8_t* mask, int64_t mask_stride_b,
                        int64_t mask_stride_m, int64_t mask_stride_r, const int32_t* seq_lens,
                        int64_t B, int64_t M, int64_t S, float scale, int dtype, void* stream) {
    return gtms::run_impl<gtms::OP_FWD>(
        in, nullptr, out, seq_lens, B, M, S, scale, dtype, GTMS_PATH_AUTO, 0u, stream,
        gtms::explicit_mask(mask, mask_stride_b, mask_stride_m, mask_stride_r));
}

int gtms_forward_masked_ex(const void* in, void* out, const uint8_t* mask,
                           int64_t mask_stride_b, int64_t mask_stride_m, int64_t mask_stride_r,
                           const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                           float scale, int dtype, int path, unsigned flags, void* stream) {
    return gtms::run_impl<gtms::OP_FWD>(
        in, nullptr, out, seq_lens, B, M, S, scale, dtype, path, flags, stream,
        gtms::explicit_mask(mask, mask_stride_b, mask_stride_m, mask_stride_r));
}

int gtms_backward_band(const void* y, const void* dy, void* dx, const int32_t* seq_lens,
                       int64_t B, int64_t M, int64_t S, int64_t lo, int64_t hi, float scale,
                       int dtype, int path, unsigned flags, void* stream) {
    return gtms::run_impl<gtms::OP_BWD>(y, dy, dx, seq_lens, B, M, S, scale, dtype, path, flags,
                                        stream, gtms::band(lo, hi));
}

int gtms_backward_masked(const void* y, const void* dy, void* dx, const uint8_t* mask,
                         int64_t mask_stride_b, int64_t mask_stride_m, int64_t mask_stride_r,
                         const int32_t* seq_lens, int64_t B, int64_t M, int64_t S, float scale,
                         int dtype, int path, unsigned flags, void* stream) {
    return gtms::run_impl<gtms::OP_BWD>(
        y, dy, dx, seq_lens, B, M, S, scale, dtype, path, flags, stream,
        gtms::explicit_mask(mask, mask_stride_b, mask_stride_m, mask_stride_r));
}

int gtms_attention_forward(const void* q, const void* k, const void* v, void* out,
                           const int32_t* seq_lens, int64_t B, int64_t M, int64_t S, int64_t D,
                           float scale, int dtype, void* stream) {
    return gtms::attention_impl(q, k, v, out, seq_lens, B, M, S, D, scale, dtype,
                                GTMS_ATTN_SPLIT_AUTO, stream);
}

int gtms_attention_forward_ex(const void* q, const void* k, const void* v, void* out,
                              const int32_t* seq_lens, int64_t B, int64_t M, int64_t S,
                              int64_t D, float scale, int dtype, int split, void* stream) {
    return gtms::attention_impl(q, k, v, out, seq_lens, B, M, S, D, scale, dtype, split, stream);
}

const char* gtms_status_string(int status) {
    switch (status) {
        case GTMS_OK: return "ok";
        case GTMS_ERR_INVALID_ARG: return "invalid argument (size, null pointer, overflow or overlap)";
        case GTMS_ERR_DTYPE: return "unknown element type";
        case GTMS_ERR_ALIGN: return "pointer not aligned to its element size";
        case GTMS_ERR_HIP: return "HIP runtime error at launch";
        case GTMS_ERR_PATH: return "kernel path unknown or unable to serve this shape";
        default: return "unknown status";
    }
}

int gtms_version(void) { return 300; }

}  // extern "C"
