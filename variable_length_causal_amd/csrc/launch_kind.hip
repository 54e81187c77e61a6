// Kernel launchers for one operation and one mask kind, chosen at compile time by
// GTMS_OP (0 forward, 1 backward) and GTMS_MK (0 tril, 1 band, 2 explicit mask).
#include "gtms.h"
#include "launch.h"
#include "backward_kernels.h"

#if !defined(GTMS_OP) || !defined(GTMS_MK)
#error "compile with -DGTMS_OP=<0|1> -DGTMS_MK=<0|1|2>"
#endif

namespace gtms {
namespace {

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

unsigned grid_for(int64_t units, int64_t per_block) {
    const int64_t blocks = cdiv(units, per_block);
    return (unsigned)(blocks < kMaxGrid ? blocks : kMaxGrid);
}

template <int OP, int MK, int DT, bool WIDE, int NV>
hipError_t launch_wave(const FwdArgs& a, hipStream_t st) {
    const dim3 grid(grid_for(a.n_units, kWaveWPB)), block(kWaveWPB * kWave);
    if constexpr (OP == OP_FWD)
        hipLaunchKernelGGL((fwd_wave<DT, WIDE, NV, kWaveWPB, kPolicyStream, MK>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((bwd_wave<DT, WIDE, NV, kWaveWPB, kPolicyStream, MK>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int OP, int MK, int DT, bool WIDE, int NV, int W>
hipError_t launch_block(const FwdArgs& a, hipStream_t st) {
    const dim3 grid(grid_for(a.n_units, 1)), block(W * kWave);
    if constexpr (OP == OP_FWD)
        hipLaunchKernelGGL((fwd_block<DT, WIDE, NV, W, kPolicyStream, MK>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((bwd_block<DT, WIDE, NV, W, kPolicyStream, MK>), grid, block, 0, st, a);
    return hipGetLastError();
}

// The backward's block path with 8 register slots per lane and an LDS stash (bwd_stash).
template <int OP, int MK, int DT, bool WIDE>
hipError_t launch_stash(const FwdArgs& a, hipStream_t st) {
    if constexpr (OP == OP_BWD && MK != MK_MASK && WIDE) {
        const dim3 grid(grid_for(a.n_units, 1)), block(kMaxW * kWave);
        hipLaunchKernelGGL((bwd_stash<DT, kAutoMaxNV, kMaxW, kPolicyStream, MK>), grid, block, 0, st, a);
        return hipGetLastError();
    } else {
        return hipErrorInvalidValue;
    }
}

template <int OP, int MK, int DT, bool WIDE>
hipError_t launch_stream(const FwdArgs& a, hipStream_t st) {
    const dim3 grid(grid_for(a.n_units, 1)), block(kStreamW * kWave);
    if constexpr (OP == OP_FWD)
        hipLaunchKernelGGL((fwd_stream<DT, WIDE, kStreamW, kPolicyStream, MK>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((bwd_stream<DT, WIDE, kStreamW, kPolicyStream, MK>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int OP, int MK, int DT, bool WIDE, int W>
hipError_t block_nv_small(int nv, const FwdArgs& a, hipStream_t st) {
    switch (nv) {
        case 1: return launch_block<OP, MK, DT, WIDE, 1, W>(a, st);
        case 2: return launch_block<OP, MK, DT, WIDE, 2, W>(a, st);
        case 4: return launch_block<OP, MK, DT, WIDE, 4, W>(a, st);
        default: return hipErrorInvalidValue;
    }
}

template <int OP, int MK, int DT, bool WIDE>
hipError_t dispatch_wide(const Plan& p, const FwdArgs& a, hipStream_t st) {
    switch (p.path) {
        case GTMS_PATH_STREAM:
            return launch_stream<OP, MK, DT, WIDE>(a, st);
        case GTMS_PATH_WAVE:
            switch (p.nv) {
                case 1: return launch_wave<OP, MK, DT, WIDE, 1>(a, st);
                case 2: return launch_wave<OP, MK, DT, WIDE, 2>(a, st);
                case 4: return launch_wave<OP, MK, DT, WIDE, 4>(a, st);
                case 8: return launch_wave<OP, MK, DT, WIDE, 8>(a, st);
                case 16: return launch_wave<OP, MK, DT, WIDE, 16>(a, st);
                default: return hipErrorInvalidValue;
            }
        default:  // block
            switch (p.w) {
                case 2: return block_nv_small<OP, MK, DT, WIDE, 2>(p.nv, a, st);
                case 4: return block_nv_small<OP, MK, DT, WIDE, 4>(p.nv, a, st);
                case 8: return block_nv_small<OP, MK, DT, WIDE, 8>(p.nv, a, st);
                default:
                    switch (p.nv) {
                        case 1: return launch_block<OP, MK, DT, WIDE, 1, 16>(a, st);
                        case 2: return launch_block<OP, MK, DT, WIDE, 2, 16>(a, st);
                        case 4: return launch_block<OP, MK, DT, WIDE, 4, 16>(a, st);
                        case 8: return launch_block<OP, MK, DT, WIDE, 8, 16>(a, st);
                        case 16:
                            if (p.stash) return launch_stash<OP, MK, DT, WIDE>(a, st);
                            return launch_block<OP, MK, DT, WIDE, 16, 16>(a, st);
                        default: return hipErrorInvalidValue;
                    }
            }
    }
}

template <int OP, int MK, int DT>
hipError_t dispatch(const Plan& p, const FwdArgs& a, hipStream_t st) {
    return p.wide ? dispatch_wide<OP, MK, DT, true>(p, a, st)
                  : dispatch_wide<OP, MK, DT, false>(p, a, st);
}

}  // namespace

template <int OP, int MK>
hipError_t launch_kind(int dtype, const Plan& p, const FwdArgs& a, hipStream_t st) {
    switch (dtype) {
        case GTMS_F32: return dispatch<OP, MK, DT_F32>(p, a, st);
        case GTMS_F16: return dispatch<OP, MK, DT_F16>(p, a, st);
        default: return dispatch<OP, MK, DT_BF16>(p, a, st);
    }
}

template hipError_t launch_kind<GTMS_OP, GTMS_MK>(int, const Plan&, const FwdArgs&, hipStream_t);

}  // namespace gtms
