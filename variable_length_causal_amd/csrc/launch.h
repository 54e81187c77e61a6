// Internal interface between the host logic (gtms_api.hip) and the kernel launchers
// (launch_kind.hip, compiled once per operation and mask kind so that the instantiations
// build in parallel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attention_kernels.h"
#include "forward_kernels.h"

namespace gtms {

constexpr int kMaxNV = 16;      // register-held vectors per lane
constexpr int kAutoNV = 4;      // vectors per lane the automatic choice aims for
constexpr int kWaveWPB = 4;     // wavefronts per workgroup on the wave path
constexpr int kMaxW = 16;       // wavefronts per workgroup on the block path, at most
constexpr int kStreamW = 8;     // wavefronts per workgroup on the stream path
constexpr int64_t kMaxGrid = int64_t(1) << 22;

// OP selects the kernel family: forward (x -> y) or backward (y, g -> dx).
enum : int { OP_FWD = 0, OP_BWD = 1 };

struct Plan {
    int path;  // GTMS_PATH_WAVE / BLOCK / STREAM
    bool wide;
    int nv;    // vectors per lane (wave, block)
    int w;     // wavefronts per row (block, stream)
};

// Launches the kernel the plan names for element type `dtype` (a GTMS_* code).
template <int OP, int MK>
hipError_t launch_kind(int dtype, const Plan& p, const FwdArgs& a, hipStream_t st);

extern template hipError_t launch_kind<OP_FWD, MK_TRIL>(int, const Plan&, const FwdArgs&, hipStream_t);
extern template hipError_t launch_kind<OP_FWD, MK_BAND>(int, const Plan&, const FwdArgs&, hipStream_t);
extern template hipError_t launch_kind<OP_FWD, MK_MASK>(int, const Plan&, const FwdArgs&, hipStream_t);
extern template hipError_t launch_kind<OP_BWD, MK_TRIL>(int, const Plan&, const FwdArgs&, hipStream_t);
extern template hipError_t launch_kind<OP_BWD, MK_BAND>(int, const Plan&, const FwdArgs&, hipStream_t);
extern template hipError_t launch_kind<OP_BWD, MK_MASK>(int, const Plan&, const FwdArgs&, hipStream_t);

// Launches the fused attention kernel for element type `dtype` (GTMS_F16 or GTMS_BF16) and
// head size D (64 or 128).
hipError_t launch_attention(int dtype, int D, const AttnArgs& a, hipStream_t st);

}  // namespace gtms
