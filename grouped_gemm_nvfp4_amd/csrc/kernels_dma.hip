// kernels_dma.hip -- the device-resident problem table's plan kernel and tile
// kernel, and the launcher of the direct-to-LDS 128 x 128 kernels (their
// instantiations live in kernels_dma_one.hip, kernels_dma_special.hip and
// kernels_dma_four.hip).  The scale mapping and MFMA operand placement are
// described in kernel_common.h.
#include "kernels_dma.h"

namespace nvfp4 {
namespace {

// Device-resident grouped launch: the table the plan kernel left in the
// workspace; workgroups past its tile total return at once.
__global__ __launch_bounds__(64) void gemm_tiled_dma_dev_kernel(const uint8_t *ws)
{
    const DevHeader hd = *(const DevHeader *)ws;
    if ((int)blockIdx.x >= hd.total_tiles)
        return;
    const DevTableView view = {hd.num_groups, (const int *)(ws + 16),
                               (const GemmDesc *)(ws + dev_desc_offset(hd.num_groups))};
    tiled_dma_tile<false, kScalesPlain, 1>(view, (int)blockIdx.x);
}

// Plan of a device-resident grouped call, one workgroup: each thread checks
// up to four consecutive problems against the one-wave kernel's contract
// (sizes >= 0, K % 128 == 0 and <= kMaxGemmK, pointers present, A and B 16-byte
// and the scales 8-byte aligned, at most 2^24 tiles), writes their GemmDesc
// and tile counts (zero when outside the contract or empty), and a
// workgroup scan (64-bit, clamped to INT32_MAX) gives the exclusive prefix.
constexpr int kPlanThreads = 1024;
__global__ __launch_bounds__(kPlanThreads) void plan_device_table_kernel(const ProblemRecord *problems, int G,
                                                                          uint8_t *ws)
{
    __shared__ long long part[kPlanThreads];
    __shared__ int bad[kPlanThreads];
    int *prefix = (int *)(ws + 16);
    GemmDesc *desc = (GemmDesc *)(ws + dev_desc_offset(G));
    const int t = threadIdx.x;
    const int per = (G + kPlanThreads - 1) / kPlanThreads; // at most 4 (G <= 4096)
    const int g0 = t * per;
    long long local[4] = {0, 0, 0, 0};
    long long sum = 0;
    int nbad = 0;
    for (int i = 0; i < per && i < 4; ++i) {
        const int g = g0 + i;
        if (g >= G)
            break;
        const ProblemRecord p = problems[g];
        bool ok = p.M >= 0 && p.N >= 0 && p.K >= 0 && p.K % 128 == 0 && p.K <= kMaxGemmK;
        const bool empty = p.M == 0 || p.N == 0;
        long long tiles = 0;
        if (ok && !empty) {
            ok = p.C != nullptr &&
                 (p.K == 0 || (p.A != nullptr && p.SFA != nullptr && p.B != nullptr && p.SFB != nullptr &&
                               ((((uintptr_t)p.A) | ((uintptr_t)p.B)) & 15) == 0 &&
                               ((((uintptr_t)p.SFA) | ((uintptr_t)p.SFB)) & 7) == 0));
            tiles = (long long)((p.M + tiled::BM - 1) / tiled::BM) * ((p.N + tiled::BN - 1) / tiled::BN);
            if (tiles > (1 << 24))
                ok = false;
        }
        if (!ok) {
            ++nbad;
            tiles = 0;
        }
        GemmDesc d;
        d.A = p.A;
        d.SFA = p.SFA;
        d.B = p.B;
        d.SFB = p.SFB;
        d.C = p.C;
        d.M = p.M;
        d.N = p.N;
        d.K = p.K;
        d.tiles_m = p.M > 0 ? (p.M + tiled::BM - 1) / tiled::BM : 1;
        desc[g] = d;
        local[i] = tiles;
        sum += tiles;
    }
    part[t] = sum;
    bad[t] = nbad;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const long long v = t >= off ? part[t - off] : 0;
        const int b = t >= off ? bad[t - off] : 0;
        __syncthreads();
        part[t] += v;
        bad[t] += b;
        __syncthreads();
    }
    long long run = part[t] - sum;
    for (int i = 0; i < per && i < 4; ++i) {
        const int g = g0 + i;
        if (g >= G)
            break;
        prefix[g] = (int)(run < 0x7fffffffLL ? run : 0x7fffffffLL);
        run += local[i];
    }
    if (t == kPlanThreads - 1) {
        const long long total = part[t];
        const int tot = (int)(total < 0x7fffffffLL ? total : 0x7fffffffLL);
        prefix[G] = tot;
        DevHeader h;
        h.num_groups = G;
        h.total_tiles = tot;
        h.invalid_groups = bad[t];
        h.reserved = 0;
        *(DevHeader *)ws = h;
    }
}

} // namespace

hipError_t launch_tiled_dma(const GroupTable &table, TileConfig cfg, hipStream_t stream)
{
    const int tiles = table.prefix[table.num_groups];
    if (tiles <= 0)
        return hipSuccess;
    // every K a multiple of the K tile; scales 16-byte aligned (blocked, moved
    // in 16-byte pieces) or 8-byte aligned
    const uintptr_t align = cfg == kTile128x128Blocked ? 15 : 7;
    bool ok = true, pairs = true;
    for (int g = 0; g < table.num_groups; ++g) {
        ok = ok && (table.g[g].K % tiled::BK) == 0 &&
             ((((uintptr_t)table.g[g].SFA) | ((uintptr_t)table.g[g].SFB)) & align) == 0;
        pairs = pairs && (table.g[g].K % (2 * tiled::BK)) == 0; // even K tile counts: scales in pairs
    }
    if (!ok)
        return hipErrorInvalidValue;
    switch (cfg) {
    case kTile128x128Blocked:
    case kTile128x128Pow2:
        return launch_dma_special(table, cfg, stream);
    case kTile128x128K4:
        return launch_dma_four_wave(table, pairs, stream);
    default:
        return launch_dma_one_wave(table, pairs, stream);
    }
}

hipError_t launch_device_table(const ProblemRecord *problems, int num_groups, int max_tiles, void *workspace,
                               hipStream_t stream)
{
    if (num_groups <= 0 || max_tiles <= 0)
        return hipSuccess;
    if (num_groups > 4 * kPlanThreads)
        return hipErrorInvalidValue;
    uint8_t *ws = (uint8_t *)workspace;
    void *pargs[] = {const_cast<ProblemRecord **>(&problems), &num_groups, &ws};
    hipError_t e = hipLaunchKernel((const void *)plan_device_table_kernel, dim3(1), dim3(kPlanThreads), pargs, 0,
                                   stream);
    if (e != hipSuccess)
        return e;
    const uint8_t *cws = ws;
    void *gargs[] = {&cws};
    return hipLaunchKernel((const void *)gemm_tiled_dma_dev_kernel, dim3((unsigned)max_tiles), dim3(64), gargs, 0,
                           stream);
}
} // namespace nvfp4
