// Internal interface between the host logic (gtms_api.hip) and the kernel launchers
// (launch_kind.hip, compiled once per operation and mask kind so that the instantiations
// build in parallel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attention_kernels.h"
#include "backward_kernels.h"
#include "forward_kernels.h"

namespace gtms {

constexpr int kMaxNV = 16;      // register-held vectors per lane
constexpr int kAutoNV = 4;      // vectors per lane the automatic choice aims for
// Vectors per lane the automatic choice takes at most on the block path; longer rows go to
// the stream path. Measured on MI355X against forced paths: at NV = 8 the block kernels beat
// the stream kernels (bfloat16 rows of 65536: forward 5930 vs 4979 GB/s, backward 6169 vs
// 4953, explicit-mask backward 5332 vs 4044); at NV = 16 a row that keeps its fp32 values
// no longer fits in the 128 registers a lane of a 16-wavefront workgroup has, and those
// spilling kernels run 1.0-3.8x slower than the stream kernels (bfloat16 rows of 98304,
// binary32 rows of 49152).
constexpr int kAutoMaxNV = 8;
// The same cap for the forward of the tril and band masks on rows of 16-byte vectors, whose
// row parts at 16 vectors keep raw vectors only (RowPart's RAW mode): 256 KB of a row, no
// spill. bfloat16 rows of 100000 ran at 5799 GB/s this way against 4521-4750 on the stream
// path. The explicit mask's and the backward's row parts still spill at 16.
constexpr int kAutoMaxNVRaw = 16;
// The backward of the computed masks on rows of 16-byte vectors goes further on the block
// path: rows of up to kAutoMaxNV * 1024 + kStashVecs vectors keep 8 vectors per lane in
// registers and the rest in LDS (bwd_stash), so that y and g cross HBM once.
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
    bool stash = false;  // block path, backward: rows past 8 vectors per lane keep the rest in LDS
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

// The automatic choice of the attention's key split (head size 64): grids of at most
// kAttnSplitBlocksPerCU (plane, query tile) blocks per compute unit, all of them resident at
// once on the whole-tile kernel (three workgroups per CU), with rows of at least
// kAttnSplitMinS. There the longest tile's chain of key blocks sets the launch's length, and
// halving it gained 14-31% on MI355X over ten such shapes (bf16 and f16 [1-3, 4-16, 2048-16384,
// 64]); with more blocks than resident slots, or shorter rows, the split lost 3-31% (one
// workgroup per CU instead of three) or gained nothing.
constexpr int64_t kAttnSplitBlocksPerCU = 3;
constexpr int kAttnSplitMinS = 2048;

// Launches the fused attention kernel for element type `dtype` (GTMS_F16 or GTMS_BF16) and
// head size D (64 or 128); split is a GTMS_ATTN_SPLIT_* choice.
hipError_t launch_attention(int dtype, int D, const AttnArgs& a, int split, hipStream_t st);

}  // namespace gtms
