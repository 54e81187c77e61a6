// C ABI of the gtms library: argument checks, kernel choice and launches.
// Declarations and the contract of every entry point are in include/gtms.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "gtms.h"
#include "forward_kernels.h"

namespace gtms {
namespace {

constexpr int kMaxNV = 16;      // register-held vectors per lane, wave and block paths
constexpr int kBlockWaves = 8;  // wavefronts per workgroup, block and stream paths
constexpr int64_t kMaxGrid = int64_t(1) << 22;

int esize_of(int dtype) { return dtype == GTMS_F32 ? 4 : 2; }

int pow2_at_least(int64_t n) {
    int p = 1;
    while (p < n) p <<= 1;
    return p;
}

// Shared argument checks; on success fills the element size and the byte count of one
// [B, M, S, S] tensor.
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
};

// Capacity (elements per row) of the register-held paths.
int64_t wave_capacity(int vec) { return int64_t(kWave) * vec * kMaxNV; }
int64_t block_capacity(int vec) { return int64_t(kWave) * kBlockWaves * vec * kMaxNV; }
// The wave path is chosen while a lane holds at most this many vectors; longer rows go
// to the block path, which spreads them over 8 wavefronts and keeps occupancy up.
constexpr int kAutoWaveNV = 4;

int make_plan(int64_t S, int dtype, bool wide, int path, Plan* p) {
    const int vec = wide ? 16 / esize_of(dtype) : 1;
    p->wide = wide;
    if (path == GTMS_PATH_AUTO) {
        if (S <= int64_t(kWave) * vec * kAutoWaveNV) path = GTMS_PATH_WAVE;
        else if (S <= block_capacity(vec)) path = GTMS_PATH_BLOCK;
        else path = GTMS_PATH_STREAM;
    }
    p->path = path;
    switch (path) {
        case GTMS_PATH_WAVE:
            if (S > wave_capacity(vec)) return GTMS_ERR_PATH;
            p->nv = pow2_at_least((S + int64_t(kWave) * vec - 1) / (int64_t(kWave) * vec));
            return GTMS_OK;
        case GTMS_PATH_BLOCK:
            if (S > block_capacity(vec)) return GTMS_ERR_PATH;
            p->nv = pow2_at_least((S + int64_t(kWave) * kBlockWaves * vec - 1) /
                                  (int64_t(kWave) * kBlockWaves * vec));
            return GTMS_OK;
        case GTMS_PATH_STREAM:
            p->nv = 0;
            return GTMS_OK;
        default:
            return GTMS_ERR_PATH;
    }
}

// ----------------------------------------------------------------- launch by template
template <int DT, bool WIDE, int NV, int POL>
hipError_t launch_wave(const FwdArgs& a, hipStream_t st) {
    const int64_t waves_per_block = kWaveBlock / kWave;
    int64_t blocks = ((int64_t)a.n_units + waves_per_block - 1) / waves_per_block;
    if (blocks > kMaxGrid) blocks = kMaxGrid;
    hipLaunchKernelGGL((fwd_wave<DT, WIDE, NV, POL>), dim3((unsigned)blocks), dim3(kWaveBlock),
                       0, st, a);
    return hipGetLastError();
}

template <int DT, bool WIDE, int NV, int POL>
hipError_t launch_block(const FwdArgs& a, hipStream_t st) {
    const int64_t blocks = (int64_t)a.n_units < kMaxGrid ? (int64_t)a.n_units : kMaxGrid;
    hipLaunchKernelGGL((fwd_block<DT, WIDE, NV, kBlockWaves, POL>), dim3((unsigned)blocks),
                       dim3(kBlockWaves * kWave), 0, st, a);
    return hipGetLastError();
}

template <int DT, bool WIDE, int POL>
hipError_t launch_stream(const FwdArgs& a, hipStream_t st) {
    const int64_t blocks = (int64_t)a.n_units < kMaxGrid ? (int64_t)a.n_units : kMaxGrid;
    hipLaunchKernelGGL((fwd_stream<DT, WIDE, kBlockWaves, POL>), dim3((unsigned)blocks),
                       dim3(kBlockWaves * kWave), 0, st, a);
    return hipGetLastError();
}

template <int DT, bool WIDE, int POL>
hipError_t dispatch_nv(const Plan& p, const FwdArgs& a, hipStream_t st) {
    if (p.path == GTMS_PATH_STREAM) return launch_stream<DT, WIDE, POL>(a, st);
    const bool wave = p.path == GTMS_PATH_WAVE;
    switch (p.nv) {
        case 1: return wave ? launch_wave<DT, WIDE, 1, POL>(a, st) : launch_block<DT, WIDE, 1, POL>(a, st);
        case 2: return wave ? launch_wave<DT, WIDE, 2, POL>(a, st) : launch_block<DT, WIDE, 2, POL>(a, st);
        case 4: return wave ? launch_wave<DT, WIDE, 4, POL>(a, st) : launch_block<DT, WIDE, 4, POL>(a, st);
        case 8: return wave ? launch_wave<DT, WIDE, 8, POL>(a, st) : launch_block<DT, WIDE, 8, POL>(a, st);
        case 16: return wave ? launch_wave<DT, WIDE, 16, POL>(a, st) : launch_block<DT, WIDE, 16, POL>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t dispatch(const Plan& p, const FwdArgs& a, bool nt, hipStream_t st) {
    if (nt) return p.wide ? dispatch_nv<DT, true, kPolicyStream>(p, a, st)
                          : dispatch_nv<DT, false, kPolicyStream>(p, a, st);
    return p.wide ? dispatch_nv<DT, true, kPolicyDefault>(p, a, st)
                  : dispatch_nv<DT, false, kPolicyDefault>(p, a, st);
}

int forward_impl(const void* in, void* out, const int32_t* seq_lens, int64_t B, int64_t M,
                 int64_t S, float scale, int dtype, int path, unsigned flags, void* stream) {
    int64_t bytes;
    bool empty;
    int st = check_common(in, out, seq_lens, B, M, S, dtype, &bytes, &empty);
    if (st != GTMS_OK) return st;
    if (path < GTMS_PATH_AUTO || path > GTMS_PATH_STREAM) return GTMS_ERR_PATH;
    if (empty) return GTMS_OK;
    if (overlap_partial(in, out, bytes)) return GTMS_ERR_INVALID_ARG;

    const int vec = 16 / esize_of(dtype);
    const bool wide = S % vec == 0 && (uintptr_t)in % 16 == 0 && (uintptr_t)out % 16 == 0;
    Plan plan;
    st = make_plan(S, dtype, wide, path, &plan);
    if (st != GTMS_OK) return st;

    FwdArgs a;
    a.x = in;
    a.y = out;
    a.seq_lens = seq_lens;
    a.M = (uint32_t)M;
    a.S = (int)S;
    a.row_bytes = (int)(S * esize_of(dtype));
    a.flags = 0;
    if (flags & GTMS_FLAG_NO_PAIR) a.flags |= F_NO_PAIR;
    if (flags & GTMS_FLAG_NO_XCD_ORDER) a.flags |= F_NO_XCD;
    a.units_per_plane = (a.flags & F_NO_PAIR) ? (uint32_t)S : (uint32_t)((S + 1) / 2);
    const int64_t units = B * M * (int64_t)a.units_per_plane;
    if (units > (int64_t)UINT32_MAX || B * M > (int64_t)UINT32_MAX) return GTMS_ERR_INVALID_ARG;
    a.n_units = (uint32_t)units;
    a.k = (float)((double)scale * 1.4426950408889634074);  // scale * log2(e)
    const bool nt = !(flags & GTMS_FLAG_CACHED_STORES);

    hipStream_t hs = (hipStream_t)stream;
    hipError_t e;
    switch (dtype) {
        case GTMS_F32: e = dispatch<DT_F32>(plan, a, nt, hs); break;
        case GTMS_F16: e = dispatch<DT_F16>(plan, a, nt, hs); break;
        default: e = dispatch<DT_BF16>(plan, a, nt, hs); break;
    }
    return e == hipSuccess ? GTMS_OK : GTMS_ERR_HIP;
}

}  // namespace
}  // namespace gtms

extern "C" {

int gtms_forward(const void* in, void* out, const int32_t* seq_lens, int64_t B, int64_t M,
                 int64_t S, float scale, int dtype, void* stream) {
    return gtms::forward_impl(in, out, seq_lens, B, M, S, scale, dtype, GTMS_PATH_AUTO, 0u,
                              stream);
}

int gtms_forward_ex(const void* in, void* out, const int32_t* seq_lens, int64_t B,
                    int64_t M, int64_t S, float scale, int dtype, int path, unsigned flags,
                    void* stream) {
    return gtms::forward_impl(in, out, seq_lens, B, M, S, scale, dtype, path, flags, stream);
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
