// api.cpp -- the C ABI declared in include/nvfp4.h.
//
// Host only: argument checks, the tile plan (per-group tile counts and their
// exclusive prefix), the by-value kernel-argument table and the launch.  The
// argument checks run before any HIP call, so they can be exercised on a
// machine without a GPU.
#include "nvfp4.h"

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <functional>
#include <map>
#include <numeric>
#include <queue>
#include <mutex>
#include <thread>
#include <tuple>
#include <utility>
#include <vector>

#include "launch.h"

namespace {

using nvfp4::GemmDesc;
using nvfp4::GroupTable;
using nvfp4::kMaxGroupsPerLaunch;
using nvfp4::TileConfig;

// Largest K of a product: the accuracy bound (NVFP4_MAX_K in nvfp4.h).
constexpr int kMaxK = NVFP4_MAX_K;
static_assert(kMaxK == nvfp4::kMaxGemmK, "the device plan kernel checks the same limit");
// Largest K of a scale-layout conversion: the conversions only move bytes;
// beyond this a matrix's offsets would leave the 31-bit range of buffer loads.
constexpr int kMaxScaleK = 1 << 24;
// Workgroups per launch: gridDim.x * 256 threads must fit in 32 bits.
constexpr long long kMaxWorkgroups = (0xffffffffll / 256);

bool empty_output(const nvfp4_problem &p) { return p.M == 0 || p.N == 0; }

nvfp4_status check_problem(const nvfp4_problem &p)
{
    if (p.M < 0 || p.N < 0 || p.K < 0)
        return NVFP4_ERROR_INVALID_VALUE;
    if (p.K % 32 != 0 || p.K > kMaxK)
        return NVFP4_ERROR_NOT_SUPPORTED;
    if (empty_output(p))
        return NVFP4_OK;
    if (p.C == nullptr)
        return NVFP4_ERROR_INVALID_VALUE;
    if (p.K > 0) {
        if (!p.A || !p.SFA || !p.B || !p.SFB)
            return NVFP4_ERROR_INVALID_VALUE;
        if ((((uintptr_t)p.A) | ((uintptr_t)p.B)) & 15)
            return NVFP4_ERROR_NOT_SUPPORTED; // packed operands: 16-byte aligned
    }
    return NVFP4_OK;
}

// A range of one problem's tiles on the wide 128 x 256 kernel, each tile's K
// split into `split` slices.
struct WideRange {
    int prob;
    int tile0, ntiles;
    int split;
};

struct Plan {
    TileConfig cfg;
    int tile_m, tile_n, split_k;
    std::vector<int> prefix; // per input group, num_groups + 1 entries
    std::vector<int> order;  // launch order of the groups (longest K first)
    std::vector<WideRange> ranges; // kWide128x256: the ranges, in launch order
    long long total_tiles;
    long long workgroups;
    long long workspace_bytes;
};

// Workgroup slots of an MI355X: 256 CUs x 4 SIMDs for one-wave workgroups.
constexpr int kWaveSlots = 1024;

// Makespan, in K tiles, of list-scheduling `per_tile` work items (in launch
// order) onto `slots` identical slots, as the hardware dispatcher does when
// each new workgroup takes the first free slot.
long long list_makespan(const std::vector<std::pair<long long, long long>> &groups, int slots)
{
    // groups: (tile count, K tiles per tile), in launch order
    std::priority_queue<long long, std::vector<long long>, std::greater<long long>> q;
    for (int i = 0; i < slots; ++i)
        q.push(0);
    long long end = 0;
    for (const auto &g : groups)
        for (long long t = 0; t < g.first; ++t) {
            long long s = q.top();
            q.pop();
            s += g.second;
            end = std::max(end, s);
            q.push(s);
        }
    return end;
}

// Workspaces for K-split launches, one per (device, stream): work on one
// stream runs in order, so a stream's calls never use its workspace
// concurrently.  hipStreamPerThread names a different stream in every host
// thread, so for it the calling thread is part of the key.  A buffer is only
// ever replaced by a larger one; replaced buffers stay allocated (a captured
// graph may still refer to them) until nvfp4_release_workspaces.
struct WorkspaceKey {
    int dev;
    hipStream_t stream;
    std::thread::id thread; // default-constructed unless stream is hipStreamPerThread
    bool operator<(const WorkspaceKey &o) const
    {
        return std::tie(dev, stream, thread) < std::tie(o.dev, o.stream, o.thread);
    }
};
struct Workspaces {
    std::mutex mu;
    std::map<WorkspaceKey, std::pair<void *, size_t>> live;
    std::vector<std::pair<int, void *>> retired;
};

Workspaces &workspaces()
{
    static Workspaces *w = new Workspaces(); // never destroyed: usable at exit
    return *w;
}

// A library workspace: the tile counters (zero), the pair slots (every one
// kPairSentinel), then the partial tiles, all at fixed offsets.  Calls leave
// the counters zero and the pair slots at the sentinel, so these states hold
// from one call to the next.
nvfp4_status get_workspace(size_t bytes, hipStream_t stream, void **out)
{
    *out = nullptr;
    if (bytes == 0)
        return NVFP4_OK;
    bytes = std::max(bytes, (size_t)nvfp4::kPartialsOffset);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return NVFP4_ERROR_LAUNCH;
    Workspaces &w = workspaces();
    std::lock_guard<std::mutex> lock(w.mu);
    WorkspaceKey key{dev, stream, std::thread::id()};
    if (stream == hipStreamPerThread)
        key.thread = std::this_thread::get_id();
    auto &e = w.live[key];
    if (e.first != nullptr && e.second >= bytes) {
        *out = e.first;
        return NVFP4_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (stream != nullptr && hipStreamIsCapturing(stream, &cs) == hipSuccess &&
        cs != hipStreamCaptureStatusNone)
        return NVFP4_ERROR_NOT_SUPPORTED; // cannot allocate inside a capture
    const size_t grown = std::max(bytes, e.second + e.second / 2);
    const size_t rounded = (grown + (1u << 20) - 1) & ~(size_t)((1u << 20) - 1);
    void *p = nullptr;
    if (hipMalloc(&p, rounded) != hipSuccess)
        return NVFP4_ERROR_LAUNCH;
    // the tile counters start at zero and the pair slots at the sentinel
    // (stream order puts this before any use)
    if (hipMemsetAsync(p, 0, (size_t)nvfp4::kCounterBytes, stream) != hipSuccess ||
        hipMemsetD32Async((hipDeviceptr_t)((char *)p + nvfp4::kCounterBytes), (int)nvfp4::kPairSentinel,
                          (size_t)(nvfp4::kPairSlotBytes / 4), stream) != hipSuccess) {
        (void)hipFree(p);
        return NVFP4_ERROR_LAUNCH;
    }
    if (e.first != nullptr)
        w.retired.emplace_back(dev, e.first);
    e = std::make_pair(p, rounded);
    *out = p;
    return NVFP4_OK;
}

// Where a launch finds its K-split state.  pairs is null where the pair
// slots are not kept (the two-slice launches then take the ticket protocol).
struct WorkspaceView {
    int *counters;
    uint32_t *pairs;
    float *partials;
};

// The view of a library workspace (or of none).
WorkspaceView library_view(void *ws)
{
    if (ws == nullptr)
        return {nullptr, nullptr, nullptr};
    char *b = (char *)ws;
    return {(int *)b, (uint32_t *)(b + nvfp4::kCounterBytes), (float *)(b + nvfp4::kPartialsOffset)};
}

// Workgroups that keep every compute unit of an MI355X busy.
constexpr int kTargetWorkgroups = 256;
// K is split only when total * 2 <= kTargetWorkgroups: within the counters
static_assert(kTargetWorkgroups / 2 <= nvfp4::kMaxSplitTiles, "split launches fit the tile counters");
constexpr int kMaxSplitK = 16;
// The 64 x 64 panel kernel is taken for M <= 64 when its launch fills at
// least this many compute units; below that the 64 x 32 stream kernel, with
// twice the tiles, keeps more of the chip busy (measured: it is faster on
// 64x2048x7168, 32x4096x4096, 64x1024x16384, 64x7168x2080; the panel kernel
// on 64x7168x16384, 1x7168x16384, 64x16384x4096).
constexpr int kPanelMinWorkgroups = 192;
// Launches of M > 64 with at most this many 128 x 128 tiles also take the
// 64-row kernels.  Measured (event means, us; 64-row route vs the one-wave or
// four-wave 128 x 128 route): 128x128x256 4.9 vs 14.2, 1024x1024x4096 16.4
// vs 35.5, 512x512x16384 18.6 vs 88.3, 512x4096x7168 46.0 vs 55.7,
// 1024x2048x16384 79.8 vs 105.3, 2048x1024x2048 23.2 vs 26.6 (128 tiles); but
// 2048x1280x4096 (160 tiles) 44.6 vs 39.8 and 2048x1536x4096 (192) 47.5 vs
// 42.4, where the four-wave form takes over.
constexpr long long kPanelMaxTiles128 = 128;

// Output tiles of every group under tile shape ts (prefix[g + 1] is the
// running total) and the longest K in K tiles.
nvfp4_status count_tiles(const nvfp4_problem *problems, int num_groups, const nvfp4::TileShape &ts,
                         std::vector<int> *prefix, long long *total, int *max_ktiles)
{
    prefix->assign(num_groups + 1, 0);
    *total = 0;
    *max_ktiles = 0;
    for (int g = 0; g < num_groups; ++g) {
        const nvfp4_problem &p = problems[g];
        long long t = 0;
        if (!empty_output(p)) {
            t = (long long)((p.M + ts.tile_m - 1) / ts.tile_m) * (long long)((p.N + ts.tile_n - 1) / ts.tile_n);
            *max_ktiles = std::max(*max_ktiles, (p.K + ts.tile_k - 1) / ts.tile_k);
        }
        *total += t;
        if (*total > kMaxWorkgroups)
            return NVFP4_ERROR_NOT_SUPPORTED;
        (*prefix)[g + 1] = (int)*total;
    }
    return NVFP4_OK;
}

// K slices per tile for the small-M kernels: split only where the tiles alone
// leave compute units idle, to at most kTargetWorkgroups workgroups in all (so
// each runs once, in a single wave of workgroups), keeping at least
// min_ktiles K tiles per slice.
int small_m_split(long long total, int max_ktiles, int min_ktiles)
{
    if (total <= 0 || total * 2 > kTargetWorkgroups)
        return 1;
    return (int)std::min<long long>(
        {kTargetWorkgroups / total, (long long)std::max(1, max_ktiles / min_ktiles), (long long)kMaxSplitK});
}

// The wide 128 x 256 tile's contract: K % 256 == 0 and 16-byte aligned scales
// in every non-empty group (A and B are 16-byte aligned in every valid call).
bool wide_ok(const nvfp4_problem *problems, int num_groups)
{
    for (int g = 0; g < num_groups; ++g) {
        const nvfp4_problem &p = problems[g];
        if (empty_output(p))
            continue;
        if (p.K % 256 != 0 || ((((uintptr_t)p.SFA) | ((uintptr_t)p.SFB)) & 15) != 0)
            return false;
    }
    return true;
}

// Wide-tile ranges of a launch (problems in plan->order, tiles counted in
// plan->prefix), balanced over the chip's CUs.  The wide workgroup holds half
// a CU (two run side by side), so the unit of balance is the CU.  Launches of
// at least kWideNoSplitTiles tiles run whole tiles only (several rounds of
// workgroups balance themselves).  Smaller ones run whole rounds of one tile
// per CU, longest K first, and split the K of the remaining tiles so that
// their work spreads over every CU: slices of about that remaining work / 256
// CUs, at least one pair of K tiles (256 K) each and at most kWideMaxSplit per
// tile.  A split whose partial tiles would take more than max_workspace
// bytes is not made.
constexpr int kCUs = 256;
constexpr long long kWideNoSplitTiles = 4LL * kCUs;
constexpr int kWideMaxSplit = nvfp4::kMaxWideSplit;
// The 64 x 128 small-M tile (one workgroup per CU) is taken with at least this
// many tiles.
constexpr long long kSkinnyMinTiles = 192;

void plan_wide_ranges(const nvfp4_problem *problems, Plan *plan, long long max_workspace)
{
    plan->ranges.clear();
    const long long T = plan->total_tiles;
    auto tiles_of = [&](int g) { return plan->prefix[g + 1] - plan->prefix[g]; };
    auto whole_only = [&]() {
        plan->ranges.clear();
        for (int g : plan->order)
            if (tiles_of(g) > 0)
                plan->ranges.push_back({g, 0, tiles_of(g), 1});
    };
    if (T >= kWideNoSplitTiles) {
        whole_only();
        return;
    }
    const long long n_whole = T / kCUs * kCUs;
    // remaining work in 32-K sub-steps, and the slice length it asks for
    long long left = n_whole, rem_work = 0;
    for (int g : plan->order) {
        const long long t = tiles_of(g);
        const long long w = std::min(t, left);
        left -= w;
        rem_work += (t - w) * (problems[g].K / 32);
    }
    const long long L = std::max(1LL, (rem_work + kCUs - 1) / kCUs);
    left = n_whole;
    long long split_tiles = 0, slots = 0;
    for (int g : plan->order) {
        const int t = tiles_of(g);
        if (t == 0)
            continue;
        const int w = (int)std::min<long long>(t, left);
        left -= w;
        if (w > 0)
            plan->ranges.push_back({g, 0, w, 1});
        if (w == t)
            continue;
        const long long k = problems[g].K / 32;
        const int s = (int)std::max(1LL, std::min({(k + L - 1) / L, (long long)kWideMaxSplit, k / 8}));
        plan->ranges.push_back({g, w, t - w, s});
        if (s > 1) {
            split_tiles += t - w;
            slots += (long long)(t - w) * s;
        }
    }
    const long long ws = slots > 0 ? nvfp4::kPartialsOffset + slots * nvfp4::kWidePartialBytes : 0;
    if (split_tiles > nvfp4::kMaxSplitTiles || ws > max_workspace)
        whole_only();
}

// Largest workspace a plan may ask for (the wide tile's balancing split).
constexpr long long kMaxPlanWorkspace = 256LL << 20;

// pow2: the power-of-two-scale path (one-wave 128 x 128 tiles on the scaled
// FP4 MFMA, no K split), which needs K % 128 == 0 and 8-byte aligned scales.
// max_workspace: the wide tile's balancing split is made only where its
// partial tiles fit in this many bytes.
nvfp4_status make_plan(const nvfp4_problem *problems, int num_groups, Plan *plan, bool pow2 = false,
                       long long max_workspace = kMaxPlanWorkspace)
{
    if (num_groups < 0 || num_groups > NVFP4_MAX_GROUPS)
        return NVFP4_ERROR_INVALID_VALUE;
    if (num_groups > 0 && problems == nullptr)
        return NVFP4_ERROR_INVALID_VALUE;
    for (int g = 0; g < num_groups; ++g) {
        nvfp4_status s = check_problem(problems[g]);
        if (s != NVFP4_OK)
            return s;
    }
    int max_m = 0;
    for (int g = 0; g < num_groups; ++g)
        if (!empty_output(problems[g]))
            max_m = std::max(max_m, problems[g].M);

    long long total = 0;
    int max_ktiles = 0;
    nvfp4_status s = NVFP4_OK;
    plan->split_k = 1;
    if (pow2) {
        for (int g = 0; g < num_groups; ++g) {
            const nvfp4_problem &p = problems[g];
            if (!empty_output(p) && (p.K % 128 != 0 || ((((uintptr_t)p.SFA) | ((uintptr_t)p.SFB)) & 7) != 0))
                return NVFP4_ERROR_NOT_SUPPORTED;
        }
        plan->cfg = nvfp4::kTile128x128Pow2;
        s = count_tiles(problems, num_groups, nvfp4::tile_shape(plan->cfg), &plan->prefix, &total, &max_ktiles);
        if (s != NVFP4_OK)
            return s;
        const nvfp4::TileShape ts = nvfp4::tile_shape(plan->cfg);
        plan->tile_m = ts.tile_m;
        plan->tile_n = ts.tile_n;
        plan->total_tiles = total;
        plan->order.resize(num_groups);
        std::iota(plan->order.begin(), plan->order.end(), 0);
        std::stable_sort(plan->order.begin(), plan->order.end(), [&](int a, int b) {
            return problems[a].K > problems[b].K;
        });
        plan->workspace_bytes = 0;
        plan->workgroups = total;
        return NVFP4_OK;
    }
    // Few 128 x 128 tiles: the 64-row kernels (eight waves per workgroup, two
    // per SIMD, K split within and across workgroups) fill the chip where one
    // wave per 128 x 128 tile would leave most SIMDs idle and run each tile's
    // K serially at the one-wave issue rate.
    bool few_tiles = false;
    if (max_m > 64) {
        std::vector<int> prefix128;
        long long total128 = 0;
        int kt128 = 0;
        s = count_tiles(problems, num_groups, nvfp4::tile_shape(nvfp4::kTile128x128), &prefix128, &total128, &kt128);
        if (s != NVFP4_OK)
            return s;
        few_tiles = total128 <= kPanelMaxTiles128;
    }
    // 32 < M <= 64 in every group, every K % 256 == 0 and aligned scales, and
    // enough columns for one 64 x 128 tile per CU without a K split: the tile
    // whose two column waves share their decoded A rows (kernels_wide.hip).
    // Measured, event means: 64 x 28672 x 4096 29.2 vs 32.7 us on the panel
    // kernel.  With a K split its 32 KiB partial tiles cost more than the panel
    // kernel's 16 KiB ones save (64 x 7168 x 16384, four slices: 35 vs 28 us),
    // so smaller launches stay on the 64-row kernels.
    bool skinny = false;
    if (max_m > 32 && max_m <= 64 && wide_ok(problems, num_groups)) {
        std::vector<int> prefix_s;
        long long total_s = 0;
        int kt_s = 0;
        s = count_tiles(problems, num_groups, nvfp4::tile_shape(nvfp4::kSkinny64x128), &prefix_s, &total_s, &kt_s);
        if (s != NVFP4_OK)
            return s;
        if (total_s >= kSkinnyMinTiles) {
            skinny = true;
            plan->cfg = nvfp4::kSkinny64x128;
            plan->split_k = 1;
            plan->prefix = prefix_s;
            total = total_s;
            max_ktiles = kt_s;
        }
    }
    if (skinny) {
        // (the ranges are set below)
    } else if (max_m > 0 && (max_m <= 64 || few_tiles)) {
        // panel: each wave takes at least one 256-K tile of a slice (8 waves)
        plan->cfg = nvfp4::kPanel64x64;
        s = count_tiles(problems, num_groups, nvfp4::tile_shape(plan->cfg), &plan->prefix, &total, &max_ktiles);
        if (s != NVFP4_OK)
            return s;
        plan->split_k = small_m_split(total, max_ktiles, 8);
        if (total * plan->split_k < kPanelMinWorkgroups) {
            // stream: a slice keeps at least 4 K tiles, half a tile per wave
            plan->cfg = nvfp4::kStream64x32;
            s = count_tiles(problems, num_groups, nvfp4::tile_shape(plan->cfg), &plan->prefix, &total, &max_ktiles);
            if (s != NVFP4_OK)
                return s;
            plan->split_k = small_m_split(total, max_ktiles, 4);
        }
    } else {
        // many tiles: the wide tile where its contract holds and it has at
        // least one tile per CU (with fewer, the partial tiles of its
        // balancing K split cost more than they save: measured 50 vs 31 us on
        // 2048 x 2048 x 2048, 128 wide tiles, against four waves per 128 x 128
        // tile), else one wave per 128 x 128 tile (or four, below)
        plan->cfg = nvfp4::kTile128x128;
        if (wide_ok(problems, num_groups)) {
            std::vector<int> prefix_w;
            long long total_w = 0;
            int kt_w = 0;
            s = count_tiles(problems, num_groups, nvfp4::tile_shape(nvfp4::kWide128x256), &prefix_w, &total_w, &kt_w);
            if (s != NVFP4_OK)
                return s;
            if (total_w >= kCUs)
                plan->cfg = nvfp4::kWide128x256;
        }
        s = count_tiles(problems, num_groups, nvfp4::tile_shape(plan->cfg), &plan->prefix, &total, &max_ktiles);
        if (s != NVFP4_OK)
            return s;
    }
    const nvfp4::TileShape ts = nvfp4::tile_shape(plan->cfg);
    plan->tile_m = ts.tile_m;
    plan->tile_n = ts.tile_n;
    plan->total_tiles = total;
    // Launch order: longest K first, so in-order dispatch is longest-first
    // (groups of equal K keep their order).
    plan->order.resize(num_groups);
    std::iota(plan->order.begin(), plan->order.end(), 0);
    std::stable_sort(plan->order.begin(), plan->order.end(), [&](int a, int b) {
        return problems[a].K > problems[b].K;
    });
    // (each of the four waves needs at least one K tile of every group)
    bool four_ok = true;
    for (int g = 0; g < num_groups; ++g)
        if (!empty_output(problems[g]) && problems[g].K < 4 * ts.tile_k)
            four_ok = false;
    if (plan->cfg == nvfp4::kTile128x128 && total > 0 && total < 4 * kWaveSlots) {
        // Fewer tiles than one-wave slots times four: compare one wave per tile
        // (kWaveSlots slots) with four waves splitting each tile's K
        // (kWaveSlots / 4 slots, a quarter of the K tiles each, plus about 3%
        // for adding the sums), both in quarter K tiles.
        std::vector<std::pair<long long, long long>> g1, g4;
        for (int gi : plan->order) {
            const nvfp4_problem &p = problems[gi];
            const long long t = plan->prefix[gi + 1] - plan->prefix[gi];
            if (t == 0)
                continue;
            const long long kt = std::max(1, (p.K + ts.tile_k - 1) / ts.tile_k);
            g1.emplace_back(t, 4 * kt);
            g4.emplace_back(t, kt + 1);
        }
        const long long m1 = list_makespan(g1, kWaveSlots);
        const long long m4 = four_ok ? list_makespan(g4, kWaveSlots / 4) * 103 / 100 : -1;
        // Measured: per K tile the four-wave form is slower than four
        // independent one-wave workgroups (the 8-group and 2-group workloads
        // ran 10-17% slower with it), so it is taken only where the model
        // promises at least a factor of two.
        if (m4 >= 0 && 2 * m4 < m1)
            plan->cfg = nvfp4::kTile128x128K4;
    }
    plan->workspace_bytes = nvfp4::workspace_bytes(plan->cfg, total, plan->split_k);
    plan->workgroups = total * plan->split_k;
    if (plan->cfg == nvfp4::kSkinny64x128) {
        // one range per problem, whole tiles
        plan->ranges.clear();
        for (int g : plan->order) {
            const int t = plan->prefix[g + 1] - plan->prefix[g];
            if (t > 0)
                plan->ranges.push_back({g, 0, t, 1});
        }
        plan->workgroups = total;
        plan->workspace_bytes = 0;
    }
    if (plan->cfg == nvfp4::kWide128x256) {
        plan_wide_ranges(problems, plan, max_workspace);
        long long slots = 0, wgs = 0;
        int max_split = 1;
        for (const WideRange &r : plan->ranges) {
            wgs += (long long)r.ntiles * r.split;
            if (r.split > 1)
                slots += (long long)r.ntiles * r.split;
            max_split = std::max(max_split, r.split);
        }
        plan->split_k = max_split;
        plan->workgroups = wgs;
        plan->workspace_bytes = slots > 0 ? nvfp4::kPartialsOffset + slots * nvfp4::kWidePartialBytes : 0;
    }
    return NVFP4_OK;
}

void fill_info(const Plan &plan, nvfp4_plan_info *info)
{
    info->kernel = plan.total_tiles == 0 ? 0
                   : plan.cfg == nvfp4::kWide128x256 ? 4
                   : plan.cfg == nvfp4::kSkinny64x128 ? 5
                   : plan.split_k > 1 ? 2
                   : plan.cfg == nvfp4::kTile128x128K4 ? 3 : 1;
    info->tile_m = plan.tile_m;
    info->tile_n = plan.tile_n;
    info->split_k = plan.split_k;
    info->total_tiles = (int)plan.total_tiles;
    info->workgroups = (int)plan.workgroups;
    info->workspace_bytes = plan.workspace_bytes;
}

// Launches a finished plan with its workspace (counters zero, partial tiles
// room for the plan's split): groups in plan order, kMaxGroupsPerLaunch per
// launch.
// blocked: SFA and SFB of every problem are in the blocked layout
nvfp4_status launch_wide_plan(const nvfp4_problem *problems, const Plan &plan, WorkspaceView ws, hipStream_t stream,
                              bool blocked = false)
{
    const nvfp4::TileShape ts = nvfp4::tile_shape(plan.cfg);
    const int bm = ts.tile_m, bn = ts.tile_n;
    nvfp4::WideTable table;
    memset(&table, 0, sizeof(table));
    table.tile_rows = bm;
    table.tile_cols = bn;
    table.blocked = blocked ? 1 : 0;
    int n = 0, cnt = 0;
    long long slot = 0;
    auto flush = [&]() -> nvfp4_status {
        if (n == 0)
            return NVFP4_OK;
        table.num_groups = n;
        table.tile_rows = bm;
        table.tile_cols = bn;
        table.blocked = blocked ? 1 : 0;
        // launches of one call share the workspace: stream order keeps them apart
        const hipError_t e = nvfp4::launch_wide(table, ws.counters, ws.partials, stream);
        n = 0;
        cnt = 0;
        slot = 0;
        return e == hipSuccess ? NVFP4_OK : NVFP4_ERROR_LAUNCH;
    };
    for (const WideRange &r : plan.ranges) {
        const nvfp4_problem &p = problems[r.prob];
        nvfp4::WideDesc &d = table.g[n];
        d.A = (const uint8_t *)p.A;
        d.SFA = (const uint8_t *)p.SFA;
        d.B = (const uint8_t *)p.B;
        d.SFB = (const uint8_t *)p.SFB;
        d.C = (uint16_t *)p.C;
        d.M = p.M;
        d.N = p.N;
        d.K = p.K;
        d.tiles_m = (p.M + bm - 1) / bm;
        d.tiles_n = (p.N + bn - 1) / bn;
        d.tile0 = r.tile0;
        d.split = r.split;
        d.cnt0 = r.split > 1 ? cnt : 0;
        d.slot0 = r.split > 1 ? (int)slot : 0;
        if (r.split > 1) {
            cnt += r.ntiles;
            slot += (long long)r.ntiles * r.split;
        }
        table.prefix[n + 1] = table.prefix[n] + r.ntiles * r.split;
        ++n;
        if (n == nvfp4::kMaxWideRanges) {
            const nvfp4_status s = flush();
            if (s != NVFP4_OK)
                return s;
        }
    }
    return flush();
}

nvfp4_status launch_plan(const nvfp4_problem *problems, const Plan &plan, WorkspaceView ws, hipStream_t stream)
{
    if (plan.cfg == nvfp4::kWide128x256 || plan.cfg == nvfp4::kSkinny64x128)
        return launch_wide_plan(problems, plan, ws, stream);
    nvfp4_status s = NVFP4_OK;
    GroupTable table;
    memset(&table, 0, sizeof(table));
    table.split_k = plan.split_k;
    // two-slice panel launches sum through the pair slots (the stream tile's
    // sixteen-byte partial stores keep the ticket protocol faster)
    const bool panel = plan.cfg == nvfp4::kPanel64x64 || plan.cfg == nvfp4::kPanel64x64Blocked;
    table.pairs = plan.split_k == 2 && panel ? ws.pairs : nullptr;
    int n = 0;
    auto flush = [&]() -> nvfp4_status {
        if (n == 0)
            return NVFP4_OK;
        table.num_groups = n;
        // launches of one call share the workspace: stream order keeps them apart
        hipError_t e = nvfp4::launch_grouped(table, plan.cfg, ws.counters, ws.partials, stream);
        n = 0;
        table.prefix[0] = 0;
        return e == hipSuccess ? NVFP4_OK : NVFP4_ERROR_LAUNCH;
    };
    for (int g : plan.order) {
        const nvfp4_problem &p = problems[g];
        const int tiles = plan.prefix[g + 1] - plan.prefix[g];
        if (tiles == 0)
            continue;
        GemmDesc &d = table.g[n];
        d.A = (const uint8_t *)p.A;
        d.SFA = (const uint8_t *)p.SFA;
        d.B = (const uint8_t *)p.B;
        d.SFB = (const uint8_t *)p.SFB;
        d.C = (uint16_t *)p.C;
        d.M = p.M;
        d.N = p.N;
        d.K = p.K;
        d.tiles_m = (p.M + plan.tile_m - 1) / plan.tile_m;
        table.prefix[n + 1] = table.prefix[n] + tiles;
        ++n;
        if (n == kMaxGroupsPerLaunch) {
            s = flush();
            if (s != NVFP4_OK)
                return s;
        }
    }
    return flush();
}

// Launches a finished plan in its stream's library-owned workspace.
nvfp4_status run_plan(const nvfp4_problem *problems, const Plan &plan, hipStream_t stream)
{
    void *workspace = nullptr;
    nvfp4_status s = get_workspace((size_t)plan.workspace_bytes, stream, &workspace);
    if (s != NVFP4_OK)
        return s;
    return launch_plan(problems, plan, library_view(workspace), stream);
}

nvfp4_status run(const nvfp4_problem *problems, int num_groups, hipStream_t stream, bool pow2 = false)
{
    Plan plan;
    nvfp4_status s = make_plan(problems, num_groups, &plan, pow2);
    if (s != NVFP4_OK || plan.total_tiles == 0)
        return s;
    return run_plan(problems, plan, stream);
}

// ---------------------------------------------------------------- blocked scales

nvfp4_status check_scale_matrix(const void *a, const void *b, int rows, int K, const void *blocked)
{
    if (rows < 0 || K < 0)
        return NVFP4_ERROR_INVALID_VALUE;
    if (K % 32 != 0 || K > kMaxScaleK)
        return NVFP4_ERROR_NOT_SUPPORTED;
    if (nvfp4::conv_workgroups(rows, K / 16) > 0x7fffffffLL)
        return NVFP4_ERROR_NOT_SUPPORTED;
    if (rows == 0 || K == 0)
        return NVFP4_OK;
    if (a == nullptr || b == nullptr)
        return NVFP4_ERROR_INVALID_VALUE;
    if (((uintptr_t)blocked) & 15)
        return NVFP4_ERROR_INVALID_VALUE; // the blocked side moves in 16-byte pieces
    return NVFP4_OK;
}

nvfp4_status convert_one(const void *src, void *dst, int rows, int K, bool to_blocked, hipStream_t stream)
{
    nvfp4_status s = check_scale_matrix(src, dst, rows, K, to_blocked ? dst : src);
    if (s != NVFP4_OK || rows == 0 || K == 0)
        return s;
    nvfp4::ScaleConvTable t;
    memset(&t, 0, sizeof(t));
    t.count = 1;
    t.to_blocked = to_blocked ? 1 : 0;
    t.src[0] = (const uint8_t *)src;
    t.dst[0] = (uint8_t *)dst;
    t.rows[0] = rows;
    t.kb[0] = K / 16;
    t.prefix[1] = (int)nvfp4::conv_workgroups(rows, K / 16);
    return nvfp4::launch_scale_conversion(t, stream) == hipSuccess ? NVFP4_OK : NVFP4_ERROR_LAUNCH;
}

// Grouped product with blocked scales.  Where the plan takes one-wave 128 x
// 128 tiles and every K is a multiple of 128, that kernel reads the blocked
// scales directly.  Otherwise the scales are converted to the plain layout in
// the stream's workspace (after the tile counters, the pair slots and whatever
// the plan's K split needs), then the plain path runs on the converted copies.
nvfp4_status run_blocked(const nvfp4_problem *problems, int num_groups, hipStream_t stream)
{
    Plan plan;
    nvfp4_status s = make_plan(problems, num_groups, &plan);
    if (s != NVFP4_OK)
        return s;
    for (int g = 0; g < num_groups; ++g) {
        const nvfp4_problem &p = problems[g];
        if (!empty_output(p) && p.K > 0 && ((((uintptr_t)p.SFA) | ((uintptr_t)p.SFB)) & 15))
            return NVFP4_ERROR_INVALID_VALUE;
    }
    if (plan.total_tiles == 0)
        return NVFP4_OK;
    if (plan.cfg == nvfp4::kWide128x256 || plan.cfg == nvfp4::kSkinny64x128) {
        // the shared-decode tiles read the blocked scales directly
        void *workspace = nullptr;
        s = get_workspace((size_t)plan.workspace_bytes, stream, &workspace);
        if (s != NVFP4_OK)
            return s;
        return launch_wide_plan(problems, plan, library_view(workspace), stream, true);
    }
    // the one-wave 128 x 128 tiles (K % 128 == 0) and the small-M panel and
    // stream tiles (K % 256 == 0) also read the blocked scales directly
    const int direct_k = plan.cfg == nvfp4::kTile128x128                                      ? 128
                         : (plan.cfg == nvfp4::kPanel64x64 || plan.cfg == nvfp4::kStream64x32) ? 256
                                                                                               : 0;
    bool direct = direct_k > 0;
    for (int g = 0; g < num_groups; ++g)
        if (direct && !empty_output(problems[g]) && problems[g].K % direct_k != 0)
            direct = false;
    if (direct) {
        plan.cfg = plan.cfg == nvfp4::kTile128x128 ? nvfp4::kTile128x128Blocked
                   : plan.cfg == nvfp4::kPanel64x64 ? nvfp4::kPanel64x64Blocked
                                                    : nvfp4::kStream64x32Blocked;
        return run_plan(problems, plan, stream);
    }
    auto up = [](long long x) { return (x + 255) & ~255LL; };
    const long long base = up(std::max<long long>(plan.workspace_bytes, nvfp4::kPartialsOffset));
    std::vector<long long> off_a(num_groups, 0), off_b(num_groups, 0);
    long long total = base;
    for (int g = 0; g < num_groups; ++g) {
        const nvfp4_problem &p = problems[g];
        if (empty_output(p) || p.K == 0)
            continue;
        off_a[g] = total;
        total += up((long long)p.M * (p.K / 16));
        off_b[g] = total;
        total += up((long long)p.N * (p.K / 16));
    }
    void *ws = nullptr;
    s = get_workspace((size_t)total, stream, &ws);
    if (s != NVFP4_OK)
        return s;
    std::vector<nvfp4_problem> plain(problems, problems + num_groups);
    nvfp4::ScaleConvTable t;
    memset(&t, 0, sizeof(t));
    auto flush = [&]() -> nvfp4_status {
        if (t.count == 0)
            return NVFP4_OK;
        const hipError_t e = nvfp4::launch_scale_conversion(t, stream);
        memset(&t, 0, sizeof(t));
        return e == hipSuccess ? NVFP4_OK : NVFP4_ERROR_LAUNCH;
    };
    for (int g = 0; g < num_groups; ++g) {
        const nvfp4_problem &p = problems[g];
        if (empty_output(p) || p.K == 0)
            continue;
        plain[g].SFA = (uint8_t *)ws + off_a[g];
        plain[g].SFB = (uint8_t *)ws + off_b[g];
        const void *srcs[2] = {p.SFA, p.SFB};
        const void *dsts[2] = {plain[g].SFA, plain[g].SFB};
        const int rows[2] = {p.M, p.N};
        for (int o = 0; o < 2; ++o) {
            const long long words = nvfp4::conv_workgroups(rows[o], p.K / 16);
            if (t.count == nvfp4::kMaxConvEntries || (long long)t.prefix[t.count] + words > 0x7fffffffLL) {
                s = flush();
                if (s != NVFP4_OK)
                    return s;
            }
            const int e = t.count++;
            t.src[e] = (const uint8_t *)srcs[o];
            t.dst[e] = (uint8_t *)dsts[o];
            t.rows[e] = rows[o];
            t.kb[e] = p.K / 16;
            t.prefix[e + 1] = t.prefix[e] + (int)words;
        }
    }
    s = flush();
    if (s != NVFP4_OK)
        return s;
    return run(plain.data(), num_groups, stream);
}

// ------------------------------------------------- allocation-free variant
//
// nvfp4_gemm_noalloc: the plan and kernels of nvfp4_gemm, with the K-split
// workspace in this file-scope device array instead of a library-allocated
// buffer.  Each GPU that runs the library holds its own copy until the
// process ends.  Host code never uses the array's name as an address: the
// device address comes from hipGetSymbolAddress, taken once per device (with
// that device current) on the entry point's first call there.
constexpr long long kScratchBytes = nvfp4::kCounterBytes + 8LL * 1024 * 1024;
static_assert(kScratchBytes == NVFP4_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchAddresses {
    std::mutex mu;
    std::map<int, void *> per_device;
};

ScratchAddresses &scratch_addresses()
{
    static ScratchAddresses *s = new ScratchAddresses(); // never destroyed: usable at exit
    return *s;
}

nvfp4_status device_scratch(void **out)
{
    *out = nullptr;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return NVFP4_ERROR_LAUNCH;
    ScratchAddresses &s = scratch_addresses();
    std::lock_guard<std::mutex> lock(s.mu);
    auto it = s.per_device.find(dev);
    if (it != s.per_device.end()) {
        *out = it->second;
        return NVFP4_OK;
    }
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
        return NVFP4_ERROR_LAUNCH;
    s.per_device[dev] = ptr;
    *out = ptr;
    return NVFP4_OK;
}

} // namespace

extern "C" {

nvfp4_status nvfp4_gemm_noalloc(const void *A, const void *SFA, const void *B, const void *SFB, void *C, int M,
                                int N, int K, hipStream_t stream)
{
    nvfp4_problem p;
    p.A = A;
    p.SFA = SFA;
    p.B = B;
    p.SFB = SFB;
    p.C = C;
    p.M = M;
    p.N = N;
    p.K = K;
    // The scratch holds the tile counters and the partial tiles; it keeps no
    // pair slots, so two-slice launches take the ticket protocol.  A plan
    // fits when its library workspace less the pair slots does.
    Plan plan;
    nvfp4_status s = make_plan(&p, 1, &plan, false, kScratchBytes + nvfp4::kPairSlotBytes);
    if (s != NVFP4_OK || plan.total_tiles == 0)
        return s;
    if (plan.workspace_bytes - nvfp4::kPairSlotBytes > kScratchBytes)
        return NVFP4_ERROR_NOT_SUPPORTED;
    WorkspaceView view{nullptr, nullptr, nullptr};
    if (plan.workspace_bytes > 0) {
        void *ws = nullptr;
        s = device_scratch(&ws);
        if (s != NVFP4_OK)
            return s;
        // the tile counters start at zero: a kernel clears them (no memset
        // node in a captured graph), ordered before the GEMM by the stream
        if (nvfp4::launch_clear_words(ws, (int)(nvfp4::kCounterBytes / 4), stream) != hipSuccess)
            return NVFP4_ERROR_LAUNCH;
        view = {(int *)ws, nullptr, (float *)((char *)ws + nvfp4::kCounterBytes)};
    }
    return launch_plan(&p, plan, view, stream);
}

nvfp4_status nvfp4_gemm(const void *A, const void *SFA, const void *B, const void *SFB,
                        void *C, int M, int N, int K, hipStream_t stream)
{
    nvfp4_problem p;
    p.A = A;
    p.SFA = SFA;
    p.B = B;
    p.SFB = SFB;
    p.C = C;
    p.M = M;
    p.N = N;
    p.K = K;
    return run(&p, 1, stream);
}

nvfp4_status nvfp4_group_gemm(const nvfp4_problem *problems, int num_groups, hipStream_t stream)
{
    return run(problems, num_groups, stream);
}

static_assert(sizeof(nvfp4::ProblemRecord) == sizeof(nvfp4_problem) &&
                  offsetof(nvfp4::ProblemRecord, C) == offsetof(nvfp4_problem, C) &&
                  offsetof(nvfp4::ProblemRecord, M) == offsetof(nvfp4_problem, M) &&
                  offsetof(nvfp4::ProblemRecord, K) == offsetof(nvfp4_problem, K),
              "the device reads nvfp4_problem as ProblemRecord");

nvfp4_status nvfp4_gemm_batched(const void *A, const void *SFA, const void *B, const void *SFB, void *C, int M,
                                int N, int K, int L, hipStream_t stream)
{
    if (L < 0 || M < 0 || N < 0 || K < 0)
        return NVFP4_ERROR_INVALID_VALUE;
    if (L > NVFP4_MAX_GROUPS)
        return NVFP4_ERROR_NOT_SUPPORTED;
    if (L == 0)
        return NVFP4_OK;
    // batch b of each operand starts b matrices into its dense stack
    const uintptr_t sa = (uintptr_t)M * (uintptr_t)(K / 2), ssa = (uintptr_t)M * (uintptr_t)(K / 16);
    const uintptr_t sb = (uintptr_t)N * (uintptr_t)(K / 2), ssb = (uintptr_t)N * (uintptr_t)(K / 16);
    const uintptr_t sc = (uintptr_t)M * (uintptr_t)N * 2;
    auto at = [](const void *base, uintptr_t step, int b) -> void * {
        return base == nullptr ? nullptr : (void *)((uintptr_t)base + step * (uintptr_t)b);
    };
    std::vector<nvfp4_problem> probs((size_t)L);
    for (int b = 0; b < L; ++b) {
        nvfp4_problem &p = probs[(size_t)b];
        p.A = at(A, sa, b);
        p.SFA = at(SFA, ssa, b);
        p.B = at(B, sb, b);
        p.SFB = at(SFB, ssb, b);
        p.C = at(C, sc, b);
        p.M = M;
        p.N = N;
        p.K = K;
    }
    return run(probs.data(), L, stream);
}

long long nvfp4_group_gemm_device_workspace_bytes(int num_groups)
{
    if (num_groups < 0 || num_groups > NVFP4_MAX_GROUPS)
        return -1;
    return nvfp4::dev_workspace_bytes(num_groups);
}

nvfp4_status nvfp4_group_gemm_device(const nvfp4_problem *problems, int num_groups, int max_tiles, void *workspace,
                                     long long workspace_bytes, hipStream_t stream)
{
    if (num_groups < 0 || num_groups > NVFP4_MAX_GROUPS || max_tiles < 0)
        return NVFP4_ERROR_INVALID_VALUE;
    if (num_groups == 0 || max_tiles == 0)
        return NVFP4_OK;
    if (problems == nullptr || workspace == nullptr || (((uintptr_t)workspace) & 15) != 0 ||
        workspace_bytes < nvfp4::dev_workspace_bytes(num_groups))
        return NVFP4_ERROR_INVALID_VALUE;
    if (max_tiles > kMaxWorkgroups)
        return NVFP4_ERROR_NOT_SUPPORTED;
    const hipError_t e = nvfp4::launch_device_table((const nvfp4::ProblemRecord *)problems, num_groups, max_tiles,
                                                    workspace, stream);
    return e == hipSuccess ? NVFP4_OK : NVFP4_ERROR_LAUNCH;
}

nvfp4_status nvfp4_gemm_pow2scale(const void *A, const void *SFA, const void *B, const void *SFB, void *C, int M,
                                  int N, int K, hipStream_t stream)
{
    nvfp4_problem p;
    p.A = A;
    p.SFA = SFA;
    p.B = B;
    p.SFB = SFB;
    p.C = C;
    p.M = M;
    p.N = N;
    p.K = K;
    return run(&p, 1, stream, true);
}

nvfp4_status nvfp4_group_gemm_pow2scale(const nvfp4_problem *problems, int num_groups, hipStream_t stream)
{
    return run(problems, num_groups, stream, true);
}

nvfp4_status nvfp4_gemm_plan(int M, int N, int K, nvfp4_plan_info *info)
{
    if (info == nullptr)
        return NVFP4_ERROR_INVALID_VALUE;
    nvfp4_problem p;
    memset(&p, 0, sizeof(p));
    p.M = M;
    p.N = N;
    p.K = K;
    // pointers are not looked at: give the checks aligned non-null stand-ins
    p.A = p.B = p.SFA = p.SFB = (const void *)(uintptr_t)256;
    p.C = (void *)(uintptr_t)256;
    Plan plan;
    nvfp4_status s = make_plan(&p, 1, &plan);
    if (s == NVFP4_OK)
        fill_info(plan, info);
    return s;
}

nvfp4_status nvfp4_group_gemm_plan(const nvfp4_problem *problems, int num_groups,
                                   nvfp4_plan_info *info, int *tile_prefix)
{
    if (info == nullptr)
        return NVFP4_ERROR_INVALID_VALUE;
    Plan plan;
    nvfp4_status s = make_plan(problems, num_groups, &plan);
    if (s != NVFP4_OK)
        return s;
    fill_info(plan, info);
    if (tile_prefix)
        for (int g = 0; g <= num_groups; ++g)
            tile_prefix[g] = plan.prefix[g];
    return NVFP4_OK;
}

long long nvfp4_blocked_scale_bytes(int rows, int K)
{
    if (rows < 0 || K < 0 || K % 32 != 0 || K > kMaxScaleK)
        return -1;
    return (long long)((rows + 127) / 128) * ((K / 16 + 3) / 4) * 512;
}

nvfp4_status nvfp4_scales_to_blocked(const void *sf, void *blocked, int rows, int K, hipStream_t stream)
{
    return convert_one(sf, blocked, rows, K, true, stream);
}

nvfp4_status nvfp4_scales_from_blocked(const void *blocked, void *sf, int rows, int K, hipStream_t stream)
{
    return convert_one(blocked, sf, rows, K, false, stream);
}

nvfp4_status nvfp4_gemm_blocked(const void *A, const void *SFA, const void *B, const void *SFB, void *C, int M,
                                int N, int K, hipStream_t stream)
{
    nvfp4_problem p;
    p.A = A;
    p.SFA = SFA;
    p.B = B;
    p.SFB = SFB;
    p.C = C;
    p.M = M;
    p.N = N;
    p.K = K;
    return run_blocked(&p, 1, stream);
}

nvfp4_status nvfp4_group_gemm_blocked(const nvfp4_problem *problems, int num_groups, hipStream_t stream)
{
    return run_blocked(problems, num_groups, stream);
}

nvfp4_status nvfp4_release_workspaces(void)
{
    Workspaces &w = workspaces();
    std::lock_guard<std::mutex> lock(w.mu);
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess)
        return NVFP4_ERROR_LAUNCH;
    nvfp4_status st = NVFP4_OK;
    auto release = [&](int dev, void *p) {
        if (hipSetDevice(dev) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
            hipFree(p) != hipSuccess)
            st = NVFP4_ERROR_LAUNCH;
    };
    for (auto &kv : w.live)
        if (kv.second.first)
            release(kv.first.dev, kv.second.first);
    for (auto &r : w.retired)
        release(r.first, r.second);
    w.live.clear();
    w.retired.clear();
    if (hipSetDevice(cur) != hipSuccess)
        st = NVFP4_ERROR_LAUNCH;
    return st;
}

const char *nvfp4_status_string(nvfp4_status status)
{
    // a C caller may pass any int: read the bits as one (an out-of-range value
    // is not a valid C++ enum value)
    static_assert(sizeof(nvfp4_status) == sizeof(int), "the status enum is an int");
    int code = 0;
    memcpy(&code, &status, sizeof(code));
    switch (code) {
    case NVFP4_OK:
        return "NVFP4_OK";
    case NVFP4_ERROR_INVALID_VALUE:
        return "NVFP4_ERROR_INVALID_VALUE: null pointer, negative size or bad group count";
    case NVFP4_ERROR_NOT_SUPPORTED:
        return "NVFP4_ERROR_NOT_SUPPORTED: K must be a multiple of 32 (at most NVFP4_MAX_K), packed "
               "operands 16-byte aligned, tile count within range";
    case NVFP4_ERROR_LAUNCH:
        return "NVFP4_ERROR_LAUNCH: a HIP launch or allocation failed";
    }
    return "unknown nvfp4_status";
}

int nvfp4_abi_version(void) { return NVFP4_ABI_VERSION; }

} // extern "C"
