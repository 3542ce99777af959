// tile_order.h -- which output tile a workgroup computes, for L2 reuse on a
// chip of eight XCDs (gfx950).
//
// Workgroups are dealt to the eight XCDs round robin in launch order, and each
// XCD has its own L2.  Inside one group of a launch the tiles r, r + 8, r +
// 16, ... (r = the tile's index in the group's range of workgroups) therefore
// run on the same XCD.
//
// Grids of at most 8 tile rows whose column count is a multiple of 8 (the
// groups of a mixture-of-experts launch) are striped: bands of 8 columns, and
// inside a band rows of 8 tiles, so every row tile of a column lands on one
// XCD and the column's B panel is fetched into one L2 only.  Measured on the
// 8-group MoE workload (N 4096, K 7168, 1 to 4 tile rows per group): 152.4 ->
// 148.5 us per launch.
//
// Larger grids give each XCD one contiguous run of a banded walk over the
// tile grid: bands of W tile columns, and inside a band rows of W tiles.  The
// workgroups an XCD holds at once then share a few rows of A and a few
// columns of B instead of touching the whole of either.
//
// Plain C++ with no HIP types, so the host tests can compile it as is.
#pragma once

#ifndef NVFP4_HD
#if defined(__HIPCC__)
#define NVFP4_HD __host__ __device__
#else
#define NVFP4_HD
#endif
#endif

namespace nvfp4 {

// Tile r (0 <= r < tiles_m * tiles_n) of a tiles_m x tiles_n grid -> (tm, tn).
// A bijection on the grid.  Other grids whose tile count is not a multiple of
// 8, or that have fewer than 64 tiles, keep the plain column-major order (tm
// fastest).
NVFP4_HD inline void tile_coords(int r, int tiles_m, int tiles_n, int *tm, int *tn)
{
    const int T = tiles_m * tiles_n;
    if ((tiles_n & 7) == 0 && tiles_m <= 8) {
        const int band = r / (8 * tiles_m), rest = r - band * 8 * tiles_m;
        *tm = rest >> 3;
        *tn = band * 8 + (rest & 7);
        return;
    }
    if (T < 64 || (T & 7) != 0) {
        *tm = r % tiles_m;
        *tn = r / tiles_m;
        return;
    }
    const int W = (tiles_n & 7) == 0 ? 8 : (tiles_n & 3) == 0 ? 4 : (tiles_n & 1) == 0 ? 2 : 1;
    const int per = T >> 3;
    const int L = (r & 7) * per + (r >> 3); // XCD part r % 8, position r / 8 within it
    const int cb = L % W;                   // column within the band
    const int rest = L / W;                 // band * tiles_m + tm
    *tm = rest % tiles_m;
    *tn = (rest / tiles_m) * W + cb;
}

} // namespace nvfp4
