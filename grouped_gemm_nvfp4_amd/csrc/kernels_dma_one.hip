// kernels_dma_one.hip -- one wave per direct-to-LDS 128 x 128 tile, plain
// [rows][K/16] scales gathered per K tile or loaded in pairs of K tiles.
#include "kernels_dma.h"

namespace nvfp4 {

hipError_t launch_dma_one_wave(const GroupTable &table, bool pairs, hipStream_t stream)
{
    const void *fn = pairs ? (const void *)gemm_tiled_dma_kernel<false, kScalesPairs>
                           : (const void *)gemm_tiled_dma_kernel<false, kScalesPlain>;
    void *args[] = {const_cast<GroupTable *>(&table)};
    return hipLaunchKernel(fn, dim3(table.prefix[table.num_groups]), dim3(64), args, 0, stream);
}
} // namespace nvfp4
