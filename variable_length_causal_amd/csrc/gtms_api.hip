// C ABI of the gtms library: argument checks, kernel choice and launches.
// Declarations and the contract of every entry point are in include/gtms.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "gtms.h"
#include "backward_kernels.h"
#include "forward_kernels.h"

namespace gtms {
namespace {

constexpr int kMaxNV = 16;      // register-held vectors per lane
constexpr int kAutoNV = 4;      // vectors per lane the automatic choice aims for
constexpr int kWaveWPB = 4;     // wavefronts per workgroup on the wave path
constexpr int kMaxW = 16;       // wavefronts per workgroup on the block path, at most
constexpr int kStreamW = 8;     // wavefronts per workgroup on the stream path
constexpr int64_t kMaxGrid = int64_t(1) << 22;
// Each XCD takes chunks of 2^4 consecutive blocks (unless GTMS_FLAG_PLAIN_ORDER). Measured on
// MI355X over chunk sizes of 1 to 4096 blocks: 16 was fastest on every workload and path
// (binary32 rows of 1000 elements four to a block, 16-bit rows of 4096 and 8192 elements one
// to a block), 4-10% above the plain round-robin order.
constexpr uint32_t kXcdChunkLog2 = 4;

int esize_of(int dtype) { return dtype == GTMS_F32 ? 4 : 2; }

int64_t pow2_at_least(int64_t n) {
    int64_t p = 1;
    while (p < n) p <<= 1;
    return p;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shared argument checks; on success fills the byte count of one [B, M, S, S] tensor.
int check_common(const void* a, const void* b, const int32_t* seq_lens, int64_t B, int64_t M,
                 int64_t S, int dtype, int64_t* bytes, bool* empty) {
    if (dtype != GTMS_F32 && dtype != GTMS_F16 && dtype != GTMS_BF16) return GTMS_ERR_DTYPE;
    if (B < 0 || M < 0 || S < 0 || S > GTMS_MAX_S || M > INT32_MAX) return GTMS_ERR_INVALID_ARG;
    int64_t n = esize_of(dtype);
    if (__builtin_mul_overflow(n, B, &n) || __builtin_mul_overflow(n, M, &n) ||
        __builtin_mul_overflow(n, S, &n) || __builtin_mul_overflow(n, S, &n))
        return GTMS_ERR_INVALID_ARG;
    *bytes = n;
    *empty = (n == 0);
    if (*empty) return GTMS_OK;
    if (!a || !b || !seq_lens) return GTMS_ERR_INVALID_ARG;
    const uintptr_t es = (uintptr_t)esize_of(dtype);
    if ((uintptr_t)a % es || (uintptr_t)b % es || (uintptr_t)seq_lens % 4) return GTMS_ERR_ALIGN;
    return GTMS_OK;
}

bool overlap_partial(const void* a, const void* b, int64_t bytes) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    if (x == y) return false;
    return x < y + (uintptr_t)bytes && y < x + (uintptr_t)bytes;
}

struct Plan {
    int path;  // GTMS_PATH_WAVE / BLOCK / STREAM
    bool wide;
    int nv;    // vectors per lane (wave, block)
    int w;     // wavefronts per row (block, stream)
};

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
// multiple of 16, else one element); a row takes 64 * W * NV slots, counting the slots it
// may write for its predecessor (line_slack).
//   auto:   rows up to 256 slots -> one wavefront per row (NV <= 4); longer rows -> W
//           wavefronts per row with NV = 4 (the stores of each instruction then cover
//           W KB of the row); W = 16 and NV up to 16 beyond that; the stream path last.
//   forced: the named path if it can hold the row.
int make_plan(int64_t S, int dtype, bool wide, int64_t slack, int path, Plan* p) {
    const int64_t vec = wide ? 16 / esize_of(dtype) : 1;
    const int64_t slots = cdiv(S, vec) + slack;  // vectors a row may span
    p->wide = wide;
    if (path == GTMS_PATH_AUTO) {
        if (slots <= kWave * kAutoNV) path = GTMS_PATH_WAVE;
        else if (slots <= int64_t(kWave) * kMaxW * kMaxNV) path = GTMS_PATH_BLOCK;
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

// ----------------------------------------------------------------- launch by template
unsigned grid_for(int64_t units, int64_t per_block) {
    const int64_t blocks = cdiv(units, per_block);
    return (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
}

// OP selects the kernel family: forward (x -> y) or backward (y, g -> dx).
enum : int { OP_FWD = 0, OP_BWD = 1 };

template <int OP, int DT, bool WIDE, int NV>
hipError_t launch_wave(const FwdArgs& a, hipStream_t st) {
    const dim3 grid(grid_for(a.n_units, kWaveWPB)), block(kWaveWPB * kWave);
    if constexpr (OP == OP_FWD)
        hipLaunchKernelGGL((fwd_wave<DT, WIDE, NV, kWaveWPB, kPolicyStream>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((bwd_wave<DT, WIDE, NV, kWaveWPB, kPolicyStream>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int OP, int DT, bool WIDE, int NV, int W>
hipError_t launch_block(const FwdArgs& a, hipStream_t st) {
    const dim3 grid(grid_for(a.n_units, 1)), block(W * kWave);
    if constexpr (OP == OP_FWD)
        hipLaunchKernelGGL((fwd_block<DT, WIDE, NV, W, kPolicyStream>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((bwd_block<DT, WIDE, NV, W, kPolicyStream>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int OP, int DT, bool WIDE>
hipError_t launch_stream(const FwdArgs& a, hipStream_t st) {
    const dim3 grid(grid_for(a.n_units, 1)), block(kStreamW * kWave);
    if constexpr (OP == OP_FWD)
        hipLaunchKernelGGL((fwd_stream<DT, WIDE, kStreamW, kPolicyStream>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((bwd_stream<DT, WIDE, kStreamW, kPolicyStream>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int OP, int DT, bool WIDE, int W>
hipError_t block_nv_small(int nv, const FwdArgs& a, hipStream_t st) {
    switch (nv) {
        case 1: return launch_block<OP, DT, WIDE, 1, W>(a, st);
        case 2: return launch_block<OP, DT, WIDE, 2, W>(a, st);
        case 4: return launch_block<OP, DT, WIDE, 4, W>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <int OP, int DT, bool WIDE>
hipError_t dispatch_wide(const Plan& p, const FwdArgs& a, hipStream_t st) {
    switch (p.path) {
        case GTMS_PATH_STREAM:
            return launch_stream<OP, DT, WIDE>(a, st);
        case GTMS_PATH_WAVE:
            switch (p.nv) {
                case 1: return launch_wave<OP, DT, WIDE, 1>(a, st);
                case 2: return launch_wave<OP, DT, WIDE, 2>(a, st);
                case 4: return launch_wave<OP, DT, WIDE, 4>(a, st);
                case 8: return launch_wave<OP, DT, WIDE, 8>(a, st);
                case 16: return launch_wave<OP, DT, WIDE, 16>(a, st);
                default: return hipErrorInvalidValue;
            }
        default:  // block
            switch (p.w) {
                case 2: return block_nv_small<OP, DT, WIDE, 2>(p.nv, a, st);
                case 4: return block_nv_small<OP, DT, WIDE, 4>(p.nv, a, st);
                case 8: return block_nv_small<OP, DT, WIDE, 8>(p.nv, a, st);
                default:
                    switch (p.nv) {
                        case 1: return launch_block<OP, DT, WIDE, 1, 16>(a, st);
                        case 2: return launch_block<OP, DT, WIDE, 2, 16>(a, st);
                        case 4: return launch_block<OP, DT, WIDE, 4, 16>(a, st);
                        case 8: return launch_block<OP, DT, WIDE, 8, 16>(a, st);
                        case 16: return launch_block<OP, DT, WIDE, 16, 16>(a, st);
                        default: return hipErrorInvalidValue;
                    }
            }
    }
}

template <int OP, int DT>
hipError_t dispatch(const Plan& p, const FwdArgs& a, hipStream_t st) {
    return p.wide ? dispatch_wide<OP, DT, true>(p, a, st) : dispatch_wide<OP, DT, false>(p, a, st);
}

// Shared body of the forward (x -> out) and backward (x = y, g = dy -> out = dx) calls.
template <int OP>
int run_impl(const void* x, const void* g, void* out, const int32_t* seq_lens, int64_t B,
             int64_t M, int64_t S, float scale, int dtype, int path, unsigned flags,
             void* stream) {
    int64_t bytes;
    bool empty;
    int st = check_common(x, out, seq_lens, B, M, S, dtype, &bytes, &empty);
    if (st != GTMS_OK) return st;
    if (path < GTMS_PATH_AUTO || path > GTMS_PATH_STREAM) return GTMS_ERR_PATH;
    if (empty) return GTMS_OK;
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
    const bool wide = S % vec == 0 && (uintptr_t)x % 16 == 0 && (uintptr_t)out % 16 == 0 &&
                      (OP == OP_FWD || (uintptr_t)g % 16 == 0);
    // whole-line writes at row boundaries (wave and block paths, rows of 16-byte vectors)
    const int64_t row_bytes = S * esize_of(dtype);
    const bool lines = wide && row_bytes >= 128 && path != GTMS_PATH_STREAM;
    Plan plan;
    st = make_plan(S, dtype, wide, line_slack(lines, row_bytes, out), path, &plan);
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
    a.units_per_plane = (a.flags & F_PAIR) ? (uint32_t)((S + 1) / 2) : (uint32_t)S;
    const int64_t units = B * M * (int64_t)a.units_per_plane;
    if (units > (int64_t)UINT32_MAX || B * M > (int64_t)UINT32_MAX) return GTMS_ERR_INVALID_ARG;
    a.n_units = (uint32_t)units;
    a.n_planes = (uint32_t)(B * M);
    // forward: scale * log2(e), so that exp is 2^x; backward: the scale itself
    a.k = OP == OP_FWD ? (float)((double)scale * 1.4426950408889634074) : scale;

    hipStream_t hs = (hipStream_t)stream;
    hipError_t e;
    switch (dtype) {
        case GTMS_F32: e = dispatch<OP, DT_F32>(plan, a, hs); break;
        case GTMS_F16: e = dispatch<OP, DT_F16>(plan, a, hs); break;
        default: e = dispatch<OP, DT_BF16>(plan, a, hs); break;
    }
    return e == hipSuccess ? GTMS_OK : GTMS_ERR_HIP;
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

int gtms_version(void) { return 100; }

}  // extern "C"
