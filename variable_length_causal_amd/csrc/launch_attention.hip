// Launcher of the fused attention kernels (one object of its own, built in parallel with
// the softmax launchers).
#include "gtms.h"
#include "attention_kernels.h"
#include "launch.h"

namespace gtms {
namespace {

// Compute units of the current device (256 on MI355X), queried once per device.
int64_t compute_units() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

}  // namespace

hipError_t launch_attention(int dtype, int D, const AttnArgs& args, int split, hipStream_t st) {
    AttnArgs a = args;
    // Block order (measured on MI355X over 10 shapes, D = 64 and 128): tile-major (longest
    // tiles of all planes first) gained 2-32% whenever the heads' K and V together fit in
    // about 3/4 of the 256 MB memory-side cache, or rows are at most 2048 long (the kernel
    // is slower there, so re-reading K and V from HBM costs less than the idle tail it
    // removes); beyond both it lost 5-13% to plane-major, which keeps a plane's K and V in
    // one XCD's L2.
    const int64_t kv_bytes = int64_t(2) * a.n_planes * a.S * D * 2;
    a.tile_major = kv_bytes <= (int64_t(192) << 20) || a.S <= 2048;
    const int64_t blocks = (int64_t)a.n_planes * a.n_tiles;
    const bool two = D == 64 && (split == GTMS_ATTN_SPLIT_ON ||
                                 (split == GTMS_ATTN_SPLIT_AUTO && a.S >= kAttnSplitMinS &&
                                  blocks <= kAttnSplitBlocksPerCU * compute_units()));
    const dim3 grid((unsigned)blocks), block(two ? 512 : 256);
    if (dtype == GTMS_BF16) {
        if (D == 128) hipLaunchKernelGGL((attn_fwd<DT_BF16, 128, 1>), grid, block, 0, st, a);
        else if (two) hipLaunchKernelGGL((attn_fwd<DT_BF16, 64, 2>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_fwd<DT_BF16, 64, 1>), grid, block, 0, st, a);
    } else {
        if (D == 128) hipLaunchKernelGGL((attn_fwd<DT_F16, 128, 1>), grid, block, 0, st, a);
        else if (two) hipLaunchKernelGGL((attn_fwd<DT_F16, 64, 2>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((attn_fwd<DT_F16, 64, 1>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace gtms
