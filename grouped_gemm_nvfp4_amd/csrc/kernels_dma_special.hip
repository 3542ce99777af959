// kernels_dma_special.hip -- one wave per direct-to-LDS 128 x 128 tile with
// scales in the blocked layout, or power-of-two scales on the FP4 MFMA.
#include "kernels_dma.h"

namespace nvfp4 {

hipError_t launch_dma_special(const GroupTable &table, TileConfig cfg, hipStream_t stream)
{
    const void *fn = cfg == kTile128x128Blocked ? (const void *)gemm_tiled_dma_kernel<false, kScalesBlocked>
                                                : (const void *)gemm_tiled_dma_kernel<true, kScalesPlain>;
    void *args[] = {const_cast<GroupTable *>(&table)};
    return hipLaunchKernel(fn, dim3(table.prefix[table.num_groups]), dim3(64), args, 0, stream);
}
} // namespace nvfp4
