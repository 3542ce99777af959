// kernels_wide.hip -- tiles whose waves share decoded A fragments through
// LDS: the 128 x 256 "wide" tile of large products and the 64 x 128 tile of
// small-M products.
//
// The scale mapping and the MFMA operand placement are those of
// kernel_common.h: each nibble and its block scale are decoded to exact fp16
// values and fed to v_mfma_f32_32x32x16_f16 with fp32 accumulation.  Decode
// VALU work per MFMA sets the speed of that mapping, so these tiles spread the
// decode over the workgroup instead of repeating it in every wave.  A tile of
// RB row blocks (32 rows each) and 64 RB columns is computed by RB column
// waves per K-group, KG K-groups per workgroup:
//
//   * column wave c owns output columns [64 c, 64 c + 64) of the tile for all
//     32 RB rows (RB x 2 MFMA blocks);
//   * it decodes its own 64 rows of B (used by no other wave) and A row block
//     c, which it shares with the other RB - 1 column waves of its K-group: it
//     keeps those fragments in registers and writes them to an LDS exchange
//     buffer, from which the others read them;
//   * per 16 K a wave decodes 3 fragments (24 VALU) for 2 RB MFMAs, where a
//     wave decoding all its own operands for the same MFMAs would decode
//     RB + 2.
//
// RB = 4, KG = 1: the 128 x 256 wide tile (four waves, 3 VALU per MFMA).
// RB = 2, KG = 4: the 64 x 128 small-M tile (eight waves; each K-group of two
// waves takes a quarter of the workgroup's K; 6 VALU per MFMA where a 64 x 64
// wave tile needs 8).  The K-groups' partial tiles are added through LDS in
// K-group order.  (The template also takes the number of column waves CW per
// K-group apart from RB, each decoding RB / CW row blocks; both tiles here
// have CW = RB.)
//
// Each wave moves only the raw rows it decodes (its 32 A rows and 64 B rows,
// plus their scales) from global memory straight into its own LDS region
// (buffer_load ... lds), two K tiles of 128 deep, so raw data needs no
// workgroup barrier.  The decoded fragments are exchanged one sub-step (32 K,
// two MFMA steps) ahead through two exchange buffers, with one LDS-only
// barrier per sub-step.  Every wave of a workgroup runs the same number of
// sub-steps (K ranges that come out shorter read zeros past their end), so
// the barriers always pair up.
//
// A launch runs ranges of tiles (WideTable in launch.h); a range may split
// each tile's K into slices, one workgroup each, for balance across the CUs.
// Each slice then stores its fp32 partial tile in the workspace and takes a
// ticket; the last one adds the partial tiles in slice order (the result does
// not depend on arrival order) and writes C.  Ordering follows the HIP / HSA
// memory model: the barrier orders every thread's partial stores before
// thread 0's release fetch-add (agent scope) on the tile's counter; the
// fetch-adds form a release sequence, so the last arriver's acquire fence
// makes all other slices' stores visible to its loads.
//
// Contract (checked by the launcher): every K % 256 == 0, SFA and SFB 16-byte
// aligned, A and B 16-byte aligned.
#include "kernel_common.h"
#include "tile_order.h"

namespace nvfp4 {
namespace {

namespace wide {
constexpr int BK = 128;
constexpr int kBRows = 64;        // the wave's own B rows
constexpr int kRowBytes = BK / 2; // 64 packed bytes per row per K tile
constexpr int kAOff = 0;          // in a stage
// scale pairs (two K tiles, 16 bytes per row): A rows in slots 0..63 (a wave
// with one A row block uses 0..31), B rows 0..63
constexpr int kPairA = 0, kPairB = 1024, kPairBytes = 2048;
constexpr int kXStep = 64 * 16; // one decoded fragment, 16 bytes per lane
constexpr int kXWave = 2 * kXStep; // one row block's fragments of a sub-step (two MFMA steps)

// RB row blocks of 32 rows, CW column waves of 64 columns per K-group, KG
// K-groups; each column wave decodes RA = RB / CW of the A row blocks.
template <int RB, int CW, int KG>
struct Shape {
    static_assert(RB % CW == 0, "each column wave decodes whole A row blocks");
    static constexpr int RA = RB / CW;
    static constexpr int BM = 32 * RB, BN = 64 * CW;
    static constexpr int kWaves = CW * KG;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int kARows = 32 * RA;                             // A rows a wave moves and decodes
    static constexpr int kBOff = kARows * kRowBytes;                   // in a stage
    static constexpr int kStageBytes = (kARows + kBRows) * kRowBytes;
    static constexpr int kWaveBytes = 2 * kStageBytes + 2 * kPairBytes;
    // load instructions per K tile: data 2 RA + 4; on even tiles the scale
    // pair, 2 plain 16-byte loads or 2 RA + 4 blocked 4-byte loads
    static constexpr int kLoadsOdd = 2 * RA + 4;
    static constexpr int kLoadsEvenPlain = kLoadsOdd + 2, kLoadsEvenBlocked = kLoadsOdd + 2 * RA + 4;
    static constexpr int kXBuf = RB * kXWave;                          // one exchange buffer of a K-group
    static constexpr int kXOff = kWaves * kWaveBytes;                  // exchange buffers [K-group][2]
    static constexpr int kLdsBytes = kXOff + (CW > 1 ? KG * 2 * kXBuf : 0);
    static constexpr int kCStride = BN * 2 + 16;                       // bytes per fp16 C row staged in LDS
    static constexpr int kAccFloats = RB * 2 * 16 * 64;                // one wave's accumulators
    static_assert(BM * kCStride <= kLdsBytes, "the C tile reuses the LDS");
    static_assert(KG == 1 || kWaves * kAccFloats * 4 <= kLdsBytes, "the K-group sums reuse the LDS");
    static_assert(kLdsBytes <= 160 * 1024, "LDS of one CU");
};
} // namespace wide

typedef __attribute__((address_space(3))) void wide_lds_void;

template <bool B>
struct EdgeTag {
    static constexpr bool value = B;
};

// s_waitcnt with only vmcnt = n (lgkmcnt and expcnt at their maxima); the
// compiler does not order the loads' LDS writes before later LDS reads, so
// nothing may move across the wait
#define WAIT_VM(n)                                                                                                   \
    do {                                                                                                             \
        asm volatile("" ::: "memory");                                                                               \
        SCHED_FENCE();                                                                                               \
        __builtin_amdgcn_s_waitcnt((((n) >> 4) << 14) | (15 << 8) | (7 << 4) | ((n) & 15));                          \
        SCHED_FENCE();                                                                                               \
        asm volatile("" ::: "memory");                                                                               \
    } while (0)
// LDS traffic done, then the workgroup barrier; the empty asm statements keep
// the compiler from moving memory accesses across it.  Loads into LDS that are
// still in flight (vmcnt) are left running.
#define LDS_BARRIER()                                                                                                \
    do {                                                                                                             \
        asm volatile("" ::: "memory");                                                                               \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                                                          \
        __builtin_amdgcn_s_barrier();                                                                                \
        asm volatile("" ::: "memory");                                                                               \
    } while (0)

// kBlocked: SFA and SFB in the blocked layout of nvfp4.h (512-byte atoms of
// 128 rows x 4 scale blocks, a 128-row tile's atoms in K order; row r, block c
// of an atom at (r % 32) * 16 + (r / 32) * 4 + c).  A row's four blocks of a
// 64-K group are then one dword of its atom: the wave fetches exactly its
// rows' dwords of the pair's four atoms (4-byte direct loads, [atom][row] in
// the pair buffer) instead of 16 contiguous bytes per row.
template <int RB, int CW, int KG, bool kBlocked>
__device__ inline void wide_tile(const WideTable &tab, const int wid, uint8_t *ws, float *parts)
{
    using namespace wide;
    using Sh = Shape<RB, CW, KG>;
    constexpr int BM = Sh::BM, BN = Sh::BN, kThreads = Sh::kThreads, RA = Sh::RA;
    constexpr int kARows = Sh::kARows, kBOff = Sh::kBOff, kStageBytes = Sh::kStageBytes;
    constexpr int kWaveBytes = Sh::kWaveBytes, kLoadsOdd = Sh::kLoadsOdd;
    constexpr int kLoadsEven = kBlocked ? Sh::kLoadsEvenBlocked : Sh::kLoadsEvenPlain;
    __shared__ __attribute__((aligned(16))) uint8_t lds[Sh::kLdsBytes];

    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int cw = wv % CW; // column wave; it decodes A row blocks RA cw .. RA cw + RA - 1
    const int kg = wv / CW; // K-group
    const int lane = (int)threadIdx.x & 63;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const uint32_t sh = h * 16;

    const int gi = find_group(tab, wid);
    const WideDesc &d = tab.g[gi];
    const int M = d.M, N = d.N, K = d.K;
    const int S = d.split;
    const int local = wid - tab.prefix[gi];
    const int tile_local = local / S, slice = local - tile_local * S;
    int tm, tn;
    tile_coords(d.tile0 + tile_local, d.tiles_m, d.tiles_n, &tm, &tn);
    const int row0 = tm * BM, col0 = tn * BN;
    const int kb_row = K / 2, ks_row = K / 16;
    // this slice's pairs of K tiles [p0, p1); K-group kg takes [q0, q1) of
    // them, every K-group running per_kg pairs (zeros past q1)
    const int npairs = K / (2 * BK);
    const int p0 = (int)((long)slice * npairs / S), p1 = (int)((long)(slice + 1) * npairs / S);
    const int per_kg = (p1 - p0 + KG - 1) / KG;
    const int q0 = min(p1, p0 + kg * per_kg), q1 = min(p1, q0 + per_kg);
    const int kt_lo = 2 * q0, nkt = 2 * q1; // K tiles with data
    const int kt_end = kt_lo + 2 * per_kg;  // K tiles the loop runs

    // this wave's rows: A [arow, arow + kARows), B [brow, brow + 64)
    const int arow = row0 + kARows * cw, brow = col0 + kBRows * cw;
    const int a_rows = max(0, min(kARows, M - arow)), b_rows = max(0, min(kBRows, N - brow));
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(d.A + (long)arow * kb_row, (uint64_t)a_rows * kb_row);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(d.B + (long)brow * kb_row, (uint64_t)b_rows * kb_row);
    // blocked scales: the 128-row tiles holding this wave's rows (whole tiles
    // of atoms; rows past M or N are the layout's zero padding) and the row
    // block of its first A and B row within them
    const int rest_k = K / 64;
    const int atile = arow / 128, btile = brow / 128;
    const int rba = (arow % 128) / 32, rbb = (brow % 128) / 32;
    const __amdgpu_buffer_rsrc_t rSA =
        kBlocked ? make_rsrc(d.SFA + (long)atile * rest_k * 512, atile < (M + 127) / 128 ? (uint64_t)rest_k * 512 : 0)
                 : make_rsrc(d.SFA + (long)arow * ks_row, (uint64_t)a_rows * ks_row);
    const __amdgpu_buffer_rsrc_t rSB =
        kBlocked ? make_rsrc(d.SFB + (long)btile * rest_k * 512, btile < (N + 127) / 128 ? (uint64_t)rest_k * 512 : 0)
                 : make_rsrc(d.SFB + (long)brow * ks_row, (uint64_t)b_rows * ks_row);

    uint8_t *const region = lds + wv * kWaveBytes;
    uint8_t *const xbase = lds + Sh::kXOff + kg * 2 * Sh::kXBuf; // this K-group's exchange buffers

    // data loads: instruction j fills rows 16 j .. 16 j + 15 of a region, lane
    // i landing at row i / 4, physical chunk i % 4, so it fetches logical chunk
    // (i % 4) ^ ((row / 4) % 4) (the swizzle `swz` of kernel_common.h)
    const int drow = lane >> 2;
    const uint32_t d_off = (uint32_t)(drow * kb_row + (((lane & 3) ^ ((drow >> 2) & 3)) << 4));
    // scale pairs: lane i -> row i, 16 bytes (A: lanes 0..31 only)
    const uint32_t pa_off = (uint32_t)(lane * ks_row);

    auto issue = [&](int st, int kt, bool pair) {
        const bool live = kt < nkt;
        uint8_t *sb = region + st * kStageBytes;
        const uint32_t kb = (uint32_t)kt * kRowBytes;
#pragma unroll
        for (int j = 0; j < 2 * RA; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (wide_lds_void *)(sb + kAOff + 1024 * j), 16,
                                                     live ? d_off + (uint32_t)(16 * j * kb_row) + kb : kOutOfRange,
                                                     0, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (wide_lds_void *)(sb + kBOff + 1024 * j), 16,
                                                     live ? d_off + (uint32_t)(16 * j * kb_row) + kb : kOutOfRange,
                                                     0, 0, 0);
        if (pair) {
            uint8_t *pb = region + 2 * kStageBytes + ((kt >> 1) & 1) * kPairBytes;
            if constexpr (kBlocked) {
                // dword idx = 64 q + lane of the pair buffer: atom j = idx / rows,
                // row r = idx % rows; the pair's atoms are 2 kt .. 2 kt + 3
#pragma unroll
                for (int q = 0; q < 2 * RA; ++q) {
                    const int idx = 64 * q + lane, j = idx / kARows, r = idx % kARows;
                    const uint32_t off = (uint32_t)((2 * kt + j) * 512 + (r % 32) * 16 + (rba + r / 32) * 4);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, (wide_lds_void *)(pb + kPairA + 256 * q), 4,
                                                             live ? off : kOutOfRange, 0, 0, 0);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int idx = 64 * q + lane, j = idx / kBRows, r = idx % kBRows;
                    const uint32_t off = (uint32_t)((2 * kt + j) * 512 + (r % 32) * 16 + (rbb + r / 32) * 4);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rSB, (wide_lds_void *)(pb + kPairB + 256 * q), 4,
                                                             live ? off : kOutOfRange, 0, 0, 0);
                }
            } else {
                const uint32_t ks = (uint32_t)kt * 8;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, (wide_lds_void *)(pb + kPairA), 16,
                                                         live && lane < kARows ? pa_off + ks : kOutOfRange, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rSB, (wide_lds_void *)(pb + kPairB), 16,
                                                         live ? pa_off + ks : kOutOfRange, 0, 0, 0);
            }
        }
    };

    // accumulators: acc[t][f] is row block (RA cw + t) % RB, column block f of
    // this wave's 64 columns; t < RA are the row blocks this wave decodes
    f32x16 acc[RB][2];
#pragma unroll
    for (int t = 0; t < RB; ++t)
#pragma unroll
        for (int f = 0; f < 2; ++f)
            acc[t][f] = (f32x16){};

    // Row blocks of the tile that hold rows of A: all RB but in a tile at the
    // M edge.  There (kEdge) the waves skip the decode, exchange and MFMAs of
    // the empty row blocks (their accumulators stay zero and are never
    // stored), so a half-empty tile costs little more than half a tile.
    const int nrb = min(RB, (M - row0 + 31) / 32);
    auto run_k = [&](auto edge_tag) {
        constexpr bool kEdge = decltype(edge_tag)::value;
        auto live_rb = [&](int i) { return !kEdge || i < nrb; };
        // raw operands of one 64-K group: this lane's 16 packed bytes of its A rows
        // and of its two B rows, and their scale words (blocks 4 g .. 4 g + 3,
        // shifted to this lane's half)
        u32x4 ra[RA], rb0, rb1;
        uint32_t wa[RA], wb0, wb1;
        auto read_raw = [&](int kt, int g) {
            const uint8_t *sb = region + (kt & 1) * kStageBytes;
            const uint8_t *pq = region + 2 * kStageBytes + ((kt >> 1) & 1) * kPairBytes;
            // the scale dword of a row for 64-K group g of tile kt
            auto scale_a = [&](int row) -> uint32_t {
                if constexpr (kBlocked)
                    return *(const uint32_t *)(pq + kPairA + ((2 * (kt & 1) + g) * kARows + row) * 4);
                else
                    return *(const uint32_t *)(pq + kPairA + 16 * row + 8 * (kt & 1) + 4 * g);
            };
            auto scale_b = [&](int row) -> uint32_t {
                if constexpr (kBlocked)
                    return *(const uint32_t *)(pq + kPairB + ((2 * (kt & 1) + g) * kBRows + row) * 4);
                else
                    return *(const uint32_t *)(pq + kPairB + 16 * row + 8 * (kt & 1) + 4 * g);
            };
#pragma unroll
            for (int r = 0; r < RA; ++r) {
                if (!live_rb(RA * cw + r))
                    continue;
                ra[r] = *(const u32x4 *)(sb + kAOff + tiled::swz(32 * r + l32, 2 * g + h));
                wa[r] = scale_a(32 * r + l32) >> sh;
            }
            rb0 = *(const u32x4 *)(sb + kBOff + tiled::swz(l32, 2 * g + h));
            rb1 = *(const u32x4 *)(sb + kBOff + tiled::swz(32 + l32, 2 * g + h));
            wb0 = scale_b(l32) >> sh;
            wb1 = scale_b(32 + l32) >> sh;
        };

        // fragments of the current sub-step (A_cur: this wave's row blocks) and of
        // the next (decoded during the current one)
        half8_t A_cur[RA][2], B_cur[2][2], A_nx[RA][2], B_nx[2][2];
        // decode this lane's fragments of half `qq` of the group in ra/rb
        auto decode = [&](int qq) {
            const half2_t cb0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb0, 1.0f, false);
            const half2_t cb1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb1, 1.0f, false);
            const half2_t sb0 = qq ? bcast_hi(cb0) : bcast_lo(cb0);
            const half2_t sb1 = qq ? bcast_hi(cb1) : bcast_lo(cb1);
#pragma unroll
            for (int r = 0; r < RA; ++r) {
                if (!live_rb(RA * cw + r))
                    continue;
                const half2_t ca = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wa[r], 1.0f, false);
                const half2_t sa = qq ? bcast_hi(ca) : bcast_lo(ca);
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    A_nx[r][s] = decode8(ra[r][2 * qq + s], sa);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                B_nx[0][s] = decode8(rb0[2 * qq + s], sb0);
                B_nx[1][s] = decode8(rb1[2 * qq + s], sb1);
            }
        };
        auto put_x = [&](int buf) {
            if constexpr (CW > 1) {
#pragma unroll
                for (int r = 0; r < RA; ++r) {
                    if (!live_rb(RA * cw + r))
                        continue;
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        *(half8_t *)(xbase + buf * Sh::kXBuf + (RA * cw + r) * kXWave + s * kXStep + lane * 16) =
                            A_nx[r][s];
                }
            }
        };


        // one sub-step (32 K): the other column waves' row blocks from exchange
        // buffer xb (read_x), then the raw read and decode of the next sub-step,
        // 2 RB x 2 MFMAs, and the next fragments into the other exchange buffer
        constexpr int kOther = RB - RA;
        half8_t Ao[kOther > 0 ? kOther : 1][2];
        auto read_x = [&](int xb) {
#pragma unroll
            for (int t = RA; t < RB; ++t) {
                if (!live_rb((RA * cw + t) % RB))
                    continue;
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    Ao[t - RA][s] = *(const half8_t *)(xbase + xb * Sh::kXBuf + ((RA * cw + t) % RB) * kXWave +
                                                       s * kXStep + lane * 16);
            }
        };
        auto mfmas = [&]() {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int t = 0; t < RA; ++t) {
                    if (!live_rb(RA * cw + t))
                        continue;
#pragma unroll
                    for (int f = 0; f < 2; ++f)
                        acc[t][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A_cur[t][s], B_cur[f][s], acc[t][f], 0, 0, 0);
                }
#pragma unroll
                for (int t = RA; t < RB; ++t) {
                    if (!live_rb((RA * cw + t) % RB))
                        continue;
#pragma unroll
                    for (int f = 0; f < 2; ++f)
                        acc[t][f] =
                            __builtin_amdgcn_mfma_f32_32x32x16_f16(Ao[t - RA][s], B_cur[f][s], acc[t][f], 0, 0, 0);
                }
            }
        };
        auto advance = [&]() {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int r = 0; r < RA; ++r)
                    if (live_rb(RA * cw + r))
                        A_cur[r][s] = A_nx[r][s];
                B_cur[0][s] = B_nx[0][s];
                B_cur[1][s] = B_nx[1][s];
            }
        };
        // the exchange needs the workgroup barrier; waves that decode all their
        // own operands (CW == 1) run on their own
        auto sync = [&]() {
            if constexpr (CW > 1)
                LDS_BARRIER();
        };

        // prologue: the range's first two K tiles in flight, the first landed, its
        // sub-step 0 decoded and exchanged
        issue(0, kt_lo, true);
        issue(1, kt_lo + 1, false);
        WAIT_VM(kLoadsOdd);
        read_raw(kt_lo, 0);
        decode(0);
        put_x(0);
        advance();
        sync();

        // sub-step u of K tile kt (u = 0..3; PAR = kt % 2), exchange buffer u % 2
        // holds its fragments.  u = 1, 3: the next group's raw operands are read
        // (u = 3: from tile kt + 1, waited for first); u = 2: tile kt + 2 is
        // issued into this tile's stage, whose last read was at u = 1.
#define WIDE_SUBSTEP(U, PAR)                                                                                         \
        do {                                                                                                             \
            read_x((U) & 1);                                                                                             \
            if ((U) == 3) {                                                                                              \
                WAIT_VM((PAR) == 0 ? kLoadsEven : kLoadsOdd);                                                            \
                read_raw(kt + 1, 0);                                                                                     \
            } else if ((U) == 1) {                                                                                       \
                read_raw(kt, 1);                                                                                         \
            }                                                                                                            \
            decode(((U) + 1) & 1);                                                                                       \
            mfmas();                                                                                                     \
            put_x(((U) + 1) & 1);                                                                                        \
            if ((U) == 2)                                                                                                \
                issue(kt & 1, kt + 2, (PAR) == 0);                                                                       \
            advance();                                                                                                   \
            sync();                                                                                                      \
        } while (0)

        for (int kt = kt_lo; kt < kt_end; kt += 2) {
            WIDE_SUBSTEP(0, 0);
            WIDE_SUBSTEP(1, 0);
            WIDE_SUBSTEP(2, 0);
            WIDE_SUBSTEP(3, 0);
            ++kt;
            WIDE_SUBSTEP(0, 1);
            WIDE_SUBSTEP(1, 1);
            WIDE_SUBSTEP(2, 1);
            WIDE_SUBSTEP(3, 1);
            --kt;
        }
#undef WIDE_SUBSTEP
    };
    if (nrb == RB)
        run_k(EdgeTag<false>{});
    else
        run_k(EdgeTag<true>{});

    // the trailing (out-of-range) loads have landed and every wave is past its
    // last LDS access
    __builtin_amdgcn_s_waitcnt(0);
    LDS_BARRIER();

    const int tid = (int)threadIdx.x;
    const long tile_slot0 = (long)d.slot0 + (long)tile_local * S;
    int *const counter = (int *)ws + d.cnt0 + tile_local;
    // last-arriver protocol of a split tile (every thread calls it after
    // storing its partial values): true in the workgroup that adds the slices
    auto last_slice = [&]() -> bool {
        __syncthreads(); // every thread's partial stores precede the ticket
        if (tid == 0) {
            const bool last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
            if (last)
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            *(volatile int *)lds = last ? 1 : 0;
        }
        __syncthreads();
        const bool last = *(volatile int *)lds != 0;
        __syncthreads(); // the flag is read before the LDS is reused
        return last;
    };

    if constexpr (KG == 1) {
        if (S > 1) {
            // partial tile of this slice: float4 q of thread t at (q kThreads
            // + t) * 16 bytes of its slot, so each store is contiguous
            float4 *mine = (float4 *)(parts + (tile_slot0 + slice) * (BM * BN));
#pragma unroll
            for (int t = 0; t < RB; ++t)
#pragma unroll
                for (int f = 0; f < 2; ++f)
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4)
                        mine[((t * 2 + f) * 4 + e4) * kThreads + tid] = (float4){
                            acc[t][f][4 * e4], acc[t][f][4 * e4 + 1], acc[t][f][4 * e4 + 2], acc[t][f][4 * e4 + 3]};
            if (!last_slice())
                return;
            // the slices in slice order, one MFMA block (16 of the thread's
            // values) at a time with the other slices' loads of it in flight
            // (at most kMaxWideSplit slices; o-th other slice: o, or o + 1 from
            // this slice on)
            constexpr int kMaxO = kMaxWideSplit - 1;
#pragma unroll
            for (int t = 0; t < RB; ++t)
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    float4 x[kMaxO][4];
#pragma unroll
                    for (int o = 0; o < kMaxO; ++o) {
                        const int j = o < slice ? o : o + 1;
                        if (j < S) {
                            const float4 *src = (const float4 *)(parts + (tile_slot0 + j) * (BM * BN));
#pragma unroll
                            for (int e4 = 0; e4 < 4; ++e4)
                                x[o][e4] = src[((t * 2 + f) * 4 + e4) * kThreads + tid];
                        }
                    }
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4) {
                        const float4 own = (float4){acc[t][f][4 * e4], acc[t][f][4 * e4 + 1], acc[t][f][4 * e4 + 2],
                                                    acc[t][f][4 * e4 + 3]};
                        float4 sum = own;
#pragma unroll
                        for (int j = 0; j < kMaxWideSplit; ++j)
                            if (j < S) {
                                const float4 v = j == slice ? own : x[j < slice ? j : j - 1][e4];
                                sum = j == 0 ? v : sum + v;
                            }
                        acc[t][f][4 * e4] = sum.x;
                        acc[t][f][4 * e4 + 1] = sum.y;
                        acc[t][f][4 * e4 + 2] = sum.z;
                        acc[t][f][4 * e4 + 3] = sum.w;
                    }
                }
            if (tid == 0)
                __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); // for the next launch
        }
        // fp16 (round to nearest even) into the LDS C tile
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            const int i = (RA * cw + t) % RB;
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 32 * i + (e >> 2) * 8 + h * 4 + (e & 3);
                    const int col = 64 * cw + 32 * f + l32;
                    *(uint16_t *)(lds + row * Sh::kCStride + col * 2) =
                        __builtin_bit_cast(uint16_t, (_Float16)acc[t][f][e]);
                }
        }
    } else {
        // the K-groups' partial tiles through LDS: wave wv's value of row block
        // i (absolute), column block f, register e, lane l at ((i * 2 + f) * 16
        // + e) * 64 + l of its slot; element E of column wave c is then held by
        // K-group g at g * CW * kAccFloats + c * kAccFloats + E
        float *red = (float *)lds;
#pragma unroll
        for (int t = 0; t < RB; ++t) {
            const int i = (RA * cw + t) % RB;
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    red[wv * Sh::kAccFloats + ((i * 2 + f) * 16 + e) * 64 + lane] = acc[t][f][e];
        }
        LDS_BARRIER();
        // thread tid: elements tid + n kThreads of the tile's CW * kAccFloats,
        // added in K-group order
        constexpr int kPer = CW * Sh::kAccFloats / kThreads;
        float v[kPer];
#pragma unroll
        for (int n = 0; n < kPer; ++n) {
            const int E = tid + n * kThreads;
            float s = red[E];
#pragma unroll
            for (int g = 1; g < KG; ++g)
                s += red[g * CW * Sh::kAccFloats + E];
            v[n] = s;
        }
        LDS_BARRIER();
        if (S > 1) {
            float *mine = parts + (tile_slot0 + slice) * (BM * BN);
#pragma unroll
            for (int n = 0; n < kPer; ++n)
                mine[tid + n * kThreads] = v[n];
            if (!last_slice())
                return;
            // the slices in slice order, four at a time with all their loads
            // in flight before the first add
            float sum[kPer];
            for (int j0 = 0; j0 < S; j0 += 4) {
                float x[4][kPer];
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int j = j0 + b;
                    if (j < S && j != slice) {
                        const float *src = parts + (tile_slot0 + j) * (BM * BN) + tid;
#pragma unroll
                        for (int n = 0; n < kPer; ++n)
                            x[b][n] = src[n * kThreads];
                    }
                }
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int j = j0 + b;
                    if (j < S) {
#pragma unroll
                        for (int n = 0; n < kPer; ++n) {
                            const float xv = j == slice ? v[n] : x[b][n];
                            sum[n] = j == 0 ? xv : sum[n] + xv;
                        }
                    }
                }
            }
#pragma unroll
            for (int n = 0; n < kPer; ++n)
                v[n] = sum[n];
            if (tid == 0)
                __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); // for the next launch
        }
        // fp16 (round to nearest even) into the LDS C tile
#pragma unroll
        for (int n = 0; n < kPer; ++n) {
            const int E = tid + n * kThreads;
            const int c = E / Sh::kAccFloats, r = E % Sh::kAccFloats;
            const int l = r & 63, e = (r >> 6) & 15, f = (r >> 10) & 1, i = r >> 11;
            const int row = 32 * i + (e >> 2) * 8 + (l >> 5) * 4 + (e & 3);
            const int col = 64 * c + 32 * f + (l & 31);
            *(uint16_t *)(lds + row * Sh::kCStride + col * 2) = __builtin_bit_cast(uint16_t, (_Float16)v[n]);
        }
    }
    LDS_BARRIER();

    // 16-byte row-contiguous stores masked to M x N
    const bool vec_ok = (N % 8 == 0) && ((((uintptr_t)d.C) & 15) == 0);
    constexpr int kSegsPerRow = BN / 8;
#pragma unroll 4
    for (int s2 = 0; s2 < BM * BN / 8 / kThreads; ++s2) {
        const int seg = s2 * kThreads + tid;
        const int row = seg / kSegsPerRow, c8 = (seg % kSegsPerRow) * 8;
        const int grow = row0 + row, gcol = col0 + c8;
        if (grow >= M || gcol >= N)
            continue;
        uint16_t *dst = d.C + (long)grow * N + gcol;
        const uint16_t *src = (const uint16_t *)(lds + row * Sh::kCStride + c8 * 2);
        if (vec_ok && gcol + 8 <= N) {
            *(u32x4 *)dst = *(const u32x4 *)src;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (gcol + e < N)
                    dst[e] = src[e];
        }
    }
}

// 128 x 256 wide tiles: four waves, two workgroups per CU
template <bool kBlocked>
__global__ __launch_bounds__(256, 2) void gemm_wide_kernel(WideTable tab, uint8_t *ws, float *parts)
{
    wide_tile<4, 4, 1, kBlocked>(tab, (int)blockIdx.x, ws, parts);
}

// 64 x 128 small-M tiles: eight waves (four K-groups of two), one workgroup per CU
template <bool kBlocked>
__global__ __launch_bounds__(512, 1) void gemm_skinny_kernel(WideTable tab, uint8_t *ws, float *parts)
{
    wide_tile<2, 2, 4, kBlocked>(tab, (int)blockIdx.x, ws, parts);
}

} // namespace

hipError_t launch_wide(const WideTable &table, void *workspace, float *partials, hipStream_t stream)
{
    const int wgs = table.prefix[table.num_groups];
    if (wgs <= 0)
        return hipSuccess;
    // 128 x 256 (wide) or 64 x 128 (small M) tiles
    const bool skinny = table.tile_rows == 64 && table.tile_cols == 128;
    if (!skinny && !(table.tile_rows == 128 && table.tile_cols == 256))
        return hipErrorInvalidValue;
    const int bm = table.tile_rows, bn = table.tile_cols, kg = skinny ? 4 : 1;
    for (int g = 0; g < table.num_groups; ++g) {
        const WideDesc &d = table.g[g];
        const int n = (table.prefix[g + 1] - table.prefix[g]) / max(1, d.split);
        if (d.K % (2 * wide::BK) != 0 || ((((uintptr_t)d.SFA) | ((uintptr_t)d.SFB)) & 15) != 0 ||
            ((((uintptr_t)d.A) | ((uintptr_t)d.B)) & 15) != 0 || d.tiles_m != (d.M + bm - 1) / bm ||
            d.tiles_n != (d.N + bn - 1) / bn || d.split < 1 || n * d.split != table.prefix[g + 1] - table.prefix[g] ||
            d.tile0 < 0 || (long long)d.tile0 + n > (long long)d.tiles_m * d.tiles_n ||
            (bm == 128 && d.split > kMaxWideSplit) ||
            (d.split > 1 && (workspace == nullptr || partials == nullptr || d.split * kg > d.K / (2 * wide::BK) ||
                             d.cnt0 < 0 ||
                             d.cnt0 + n > kMaxSplitTiles || d.slot0 < 0)))
            return hipErrorInvalidValue;
    }
    uint8_t *ws = (uint8_t *)workspace;
    void *args[] = {const_cast<WideTable *>(&table), &ws, &partials};
    if (table.blocked != 0 && table.blocked != 1)
        return hipErrorInvalidValue;
    const bool blocked = table.blocked == 1;
    const void *fn = skinny ? (blocked ? (const void *)gemm_skinny_kernel<true> : (const void *)gemm_skinny_kernel<false>)
                            : (blocked ? (const void *)gemm_wide_kernel<true> : (const void *)gemm_wide_kernel<false>);
    return hipLaunchKernel(fn, dim3((unsigned)wgs), dim3(skinny ? 512 : 256), args, 0, stream);
}

} // namespace nvfp4
