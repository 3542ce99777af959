// launch.h -- what the host side hands the gfx950 kernels.
//
// Internal to the library: shared by the C-ABI layer (api.cpp) and the
// kernels (kernels.hip).  Everything travels to the device by value in the
// kernel-argument segment, so a launch needs no host-to-device copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

// One problem as the kernels see it.
struct GemmDesc {
    const uint8_t *A;   // [M][K/2] packed e2m1, low nibble = even k
    const uint8_t *SFA; // [M][K/16] e4m3
    const uint8_t *B;   // [N][K/2]
    const uint8_t *SFB; // [N][K/16]
    uint16_t *C;        // [M][N] binary16
    int M, N, K;
    int tiles_m;        // ceil(M / tile_m)
};

// Largest K of a product (NVFP4_MAX_K of the C ABI): the accuracy bound.
constexpr int kMaxGemmK = 1 << 17;

// Groups per launch.  The table below stays under the 4 KiB kernel-argument
// budget; a call with more groups is issued as several launches.
constexpr int kMaxGroupsPerLaunch = 64;

// Exclusive prefix over per-group tile counts: workgroup w (< prefix[n]) works
// on group g with prefix[g] <= w < prefix[g+1].
struct GroupTable {
    int num_groups;
    int split_k;                         // K slices per tile (1: no split)
    // split_k == 2 on the 64 x 64 panel kernel: the pair slots of the
    // workspace (kPairSlotBytes, every slot holding kPairSentinel between
    // launches), or null for the ticket protocol; other kernels ignore it
    uint32_t *pairs;
    int prefix[kMaxGroupsPerLaunch + 1]; // in output tiles
    GemmDesc g[kMaxGroupsPerLaunch];
};
static_assert(sizeof(GroupTable) <= 4096, "kernel-argument budget");

// Device-resident grouped calls: the problem table lives in device memory
// (written there by the caller, possibly by an earlier kernel), so the host
// knows neither sizes nor tile counts.  A one-workgroup plan kernel turns it
// into this table in the caller's workspace: a header, the exclusive prefix
// over per-group tile counts (num_groups + 1 ints from byte 16), then one
// GemmDesc per group from dev_desc_offset(num_groups).
struct DevHeader {
    int num_groups;
    int total_tiles;    // tiles the table asks for (clamped to INT32_MAX)
    int invalid_groups; // groups outside the contract, given no tiles
    int reserved;
};
// Layout of nvfp4_problem as the device reads it.
struct ProblemRecord {
    const uint8_t *A;
    const uint8_t *SFA;
    const uint8_t *B;
    const uint8_t *SFB;
    uint16_t *C;
    int M, N, K;
};
__host__ __device__ inline long long dev_desc_offset(int num_groups) { return (16 + 4LL * (num_groups + 1) + 15) / 16 * 16; }
inline long long dev_workspace_bytes(int num_groups)
{
    return dev_desc_offset(num_groups) + (long long)num_groups * (long long)sizeof(GemmDesc);
}
// Plan kernel, then one-wave 128 x 128 tiles over a grid of max_tiles
// workgroups (those past the table's total return at once).
hipError_t launch_device_table(const ProblemRecord *problems, int num_groups, int max_tiles, void *workspace,
                               hipStream_t stream);

// Tile configurations the kernels are built for.
enum TileConfig : int {
    kTile128x128 = 0,   // one wave per workgroup owning the whole 128 x 128 tile
    kStream64x32 = 1,   // 8 waves split K; each streams its own share; K may be split
    kTile128x128K4 = 2, // 128 x 128 tile, four waves splitting its K, sums added in LDS
    kPanel64x64 = 3,    // 8 waves split K, each owning the 64 x 64 tile; K may be split
    kTile128x128Pow2 = 5, // one-wave 128 x 128 tiles on the scaled FP4 MFMA (power-of-two scales)
    kTile128x128Blocked = 6, // one-wave 128 x 128 direct-to-LDS tiles, scales in the blocked layout
    kWide128x256 = 7,   // four waves share a 128 x 256 tile, decoded A exchanged through LDS
    kSkinny64x128 = 8,  // eight waves (4 K-groups of 2) share a 64 x 128 tile, decoded A exchanged
    kPanel64x64Blocked = 9, // kPanel64x64 reading scales in the blocked layout (every K % 256 == 0)
    kStream64x32Blocked = 10, // kStream64x32 reading scales in the blocked layout (every K % 256 == 0)
};

struct TileShape {
    int tile_m, tile_n, tile_k;
};

inline TileShape tile_shape(TileConfig c)
{
    switch (c) {
    case kStream64x32:
    case kStream64x32Blocked:
        return {64, 32, 256};
    case kPanel64x64:
    case kPanel64x64Blocked:
        return {64, 64, 256};
    case kWide128x256:
        return {128, 256, 256};
    case kSkinny64x128:
        return {64, 128, 256};
    case kTile128x128K4:
    case kTile128x128Pow2:
    case kTile128x128Blocked:
    case kTile128x128:
    default:
        return {128, 128, 128};
    }
}

// fp32 elements of one output tile's partial sum (K-split kernels).
inline long long partial_elems(TileConfig c)
{
    const TileShape t = tile_shape(c);
    return (long long)t.tile_m * t.tile_n;
}

// Device workspace of a K-split launch (bytes): kMaxSplitTiles tile counters
// (zero when the workspace is allocated; a kernel that uses them leaves them
// zero), the pair slots of two-slice launches on the panel kernel (one
// 32-bit slot per output element of at most 128 tiles of 64 x 64, each
// holding kPairSentinel between launches), then the fp32 partial tiles of
// every (tile, K slice).  Such launches have at most kMaxSplitTiles tiles.
constexpr int kMaxSplitTiles = 4096;
constexpr long long kCounterBytes = kMaxSplitTiles * 4;
constexpr long long kPairSlotBytes = 128LL * 64 * 64 * 4;
// A signalling-NaN pattern: fp32 arithmetic never produces it (NaN results
// are quiet), so no partial sum can be mistaken for an empty slot.
constexpr uint32_t kPairSentinel = 0x7FBADBADu;
constexpr long long kPartialsOffset = kCounterBytes + kPairSlotBytes;
inline long long workspace_bytes(TileConfig c, long long total_tiles, int split_k)
{
    return split_k > 1 ? kPartialsOffset + total_tiles * split_k * partial_elems(c) * 4 : 0;
}

// Launches one grouped pass (table already filled, prefix included).  A
// K-split launch takes its tile counters at `counters` and its partial tiles
// at `partials` (and its pair slots at table.pairs, when set).
hipError_t launch_grouped(const GroupTable &table, TileConfig cfg, int *counters, float *partials,
                          hipStream_t stream);
// The direct-to-LDS 128 x 128 kernels (kernels_dma.hip): one wave per tile
// (kTile128x128, kTile128x128Pow2, kTile128x128Blocked) or four
// (kTile128x128K4).  Every K % 128 == 0 and the scales 8-byte aligned
// (16-byte for blocked scales), else hipErrorInvalidValue.
hipError_t launch_tiled_dma(const GroupTable &table, TileConfig cfg, hipStream_t stream);
// Its parts, one source each (checked arguments, at least one tile): plain
// scales one wave per tile, gathered or in pairs of K tiles; blocked or
// power-of-two scales; four waves per tile.
hipError_t launch_dma_one_wave(const GroupTable &table, bool pairs, hipStream_t stream);
hipError_t launch_dma_special(const GroupTable &table, TileConfig cfg, hipStream_t stream);
hipError_t launch_dma_four_wave(const GroupTable &table, bool pairs, hipStream_t stream);
// The 128 x 256 wide tile (kernels_wide.hip).  A launch runs ranges of tiles:
// tiles [tile0, tile0 + n) of one problem's grid, each tile's K split into
// `split` slices (one workgroup each; 1 = whole K).  Slice j of the range's
// tile i is workgroup prefix[g] + i * split + j.  With split > 1 every slice
// stores its fp32 partial tile in partial slot slot0 + i * split + j of the
// workspace and takes a ticket from counter cnt0 + i; the last adds the
// slices in slice order and writes C.
struct WideDesc {
    const uint8_t *A, *SFA, *B, *SFB;
    uint16_t *C;
    int M, N, K;
    int tiles_m, tiles_n; // ceil(M / 128), ceil(N / 256)
    int tile0;            // first tile of the range (banded order of tile_order.h)
    int split;            // K slices per tile
    int cnt0, slot0;      // split > 1: first counter and first partial slot of the range
};
constexpr int kMaxWideRanges = 48;
// Largest K split of a 128 x 256 tile (the kernel adds at most this many slices).
constexpr int kMaxWideSplit = 4;
struct WideTable {
    int num_groups; // ranges in this launch
    int tile_rows;  // 128 (the wide tile) or 64 (the small-M tile)
    int tile_cols;  // 256 or 128
    int blocked;    // 1: SFA and SFB in the blocked layout (512-byte atoms), 0: [rows][K/16]
    int prefix[kMaxWideRanges + 1]; // workgroups before each range
    WideDesc g[kMaxWideRanges];
};
static_assert(sizeof(WideTable) <= 4096, "kernel-argument budget");
// one fp32 partial tile of a 128 x 256 and of a 64 x 128 tile
constexpr long long kWidePartialBytes = 128LL * 256 * 4;
constexpr long long kSkinnyPartialBytes = 64LL * 128 * 4;
// Checks the contract (every K % 256 == 0; A, B, SFA, SFB 16-byte aligned;
// the grid sizes; a workspace when some range splits) and launches.  The
// tile counters are at `workspace`, the partial tiles at `partials`.
hipError_t launch_wide(const WideTable &table, void *workspace, float *partials, hipStream_t stream);

// Scale-layout conversion, batched: entry e moves the scales of a
// rows[e] x (kb[e] = K/16) matrix between the plain [rows][K/16] layout and
// the blocked one (512-byte atoms of 128 rows x 4 blocks; byte of row m,
// block j at ((m / 128) * ceil(kb / 4) + j / 4) * 512 + (m % 32) * 16 +
// ((m / 32) % 4) * 4 + j % 4; padding rows and blocks are zero).  One
// workgroup per 128-row tile and run of kConvAtoms atoms; prefix[e] =
// workgroups of the entries before e.
constexpr int kMaxConvEntries = 128;
constexpr int kConvAtoms = 8;
struct ScaleConvTable {
    int count;
    int to_blocked; // 1: plain -> blocked (padding written as zero); 0: blocked -> plain
    int prefix[kMaxConvEntries + 1];
    const uint8_t *src[kMaxConvEntries];
    uint8_t *dst[kMaxConvEntries];
    int rows[kMaxConvEntries];
    int kb[kMaxConvEntries];
};
static_assert(sizeof(ScaleConvTable) <= 4096, "kernel-argument budget");

// Workgroups of one entry.
inline long long conv_workgroups(int rows, int kb)
{
    const long long rest_k = (kb + 3) / 4;
    return (rows + 127LL) / 128 * ((rest_k + kConvAtoms - 1) / kConvAtoms);
}

hipError_t launch_scale_conversion(const ScaleConvTable &table, hipStream_t stream);

// Sets `words` 32-bit words at p to zero with a kernel (one workgroup).
hipError_t launch_clear_words(void *p, int words, hipStream_t stream);

} // namespace nvfp4
