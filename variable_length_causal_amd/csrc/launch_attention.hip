// Launcher of the fused attention kernels (one object of its own, built in parallel with
// the softmax launchers).
#include "gtms.h"
#include "attention_kernels.h"
#include "launch.h"

namespace gtms {

hipError_t launch_attention(int dtype, int D, const AttnArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((uint64_t)a.n_planes * (uint64_t)a.n_tiles)), block(256);
    if (dtype == GTMS_BF16) {
        if (D == 64) hipLaunchKernelGGL((attn_fwd<DT_BF16, 64>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_fwd<DT_BF16, 128>), grid, block, 0, st, a);
    } else {
        if (D == 64) hipLaunchKernelGGL((attn_fwd<DT_F16, 64>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_fwd<DT_F16, 128>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace gtms
