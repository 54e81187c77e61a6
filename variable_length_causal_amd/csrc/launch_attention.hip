// Launcher of the fused attention kernels (one object of its own, built in parallel with
// the softmax launchers).
#include "gtms.h"
#include "attention_kernels.h"
#include "launch.h"

namespace gtms {

hipError_t launch_attention(int dtype, int D, const AttnArgs& args, hipStream_t st) {
    AttnArgs a = args;
    // Block order (measured on MI355X over 10 shapes, D = 64 and 128): tile-major (longest
    // tiles of all planes first) gained 2-32% whenever the heads' K and V together fit in
    // about 3/4 of the 256 MB memory-side cache, or rows are at most 2048 long (the kernel
    // is slower there, so re-reading K and V from HBM costs less than the idle tail it
    // removes); beyond both it lost 5-13% to plane-major, which keeps a plane's K and V in
    // one XCD's L2.
    const int64_t kv_bytes = int64_t(2) * a.n_planes * a.S * D * 2;
    a.tile_major = kv_bytes <= (int64_t(192) << 20) || a.S <= 2048;
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
