// kernels_dma_four.hip -- four waves per direct-to-LDS 128 x 128 tile, each
// over a quarter of its K.
#include "kernels_dma.h"

namespace nvfp4 {

hipError_t launch_dma_four_wave(const GroupTable &table, bool pairs, hipStream_t stream)
{
    const void *fn = pairs ? (const void *)gemm_tiled_dma4_kernel<kScalesPairs>
                           : (const void *)gemm_tiled_dma4_kernel<kScalesPlain>;
    void *args[] = {const_cast<GroupTable *>(&table)};
    return hipLaunchKernel(fn, dim3(table.prefix[table.num_groups]), dim3(256), args, 0, stream);
}
} // namespace nvfp4
