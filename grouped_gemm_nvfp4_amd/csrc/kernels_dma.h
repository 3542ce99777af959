// kernels_dma.h -- the gfx950 (CDNA4) NVFP4 GEMM kernels whose 128 x 128 tiles
// load straight from global memory into LDS (buffer_load ... lds), as
// templates: one wave per tile (plain, paired, blocked or power-of-two scales)
// and four waves per tile.  Each instantiation costs tens of seconds of
// compile time, so they are spread over several sources (kernels_dma*.hip)
// that compile in parallel.  The scale mapping and MFMA operand placement are
// described in kernel_common.h.
#pragma once

#include "kernel_common.h"

namespace nvfp4 {
namespace {

// ----------------------------------------------------------------------------
// One-wave 128 x 128 tile kernel with direct global -> LDS loads (gfx950
// buffer_load ... lds, 16 bytes per lane for A and B, 4 for the scales): no
// register staging slot, so the registers it would hold go to the compute.
// Two LDS stages in one array: tile kt + 1 streams into one while tile kt is
// computed from the other, with explicit waits (below).  The 16-byte chunk
// swizzle of the register-staged kernel is kept by choosing each lane's
// global chunk: a load instruction fills 16 rows of 64 bytes, lane i landing
// at row i / 4, physical chunk i % 4, so it fetches logical chunk (i % 4) ^
// ((row / 4) % 4).  Vector path only (K % 128 == 0, 8-byte aligned scales).
//
// kPow2: every scale is a power of two, E4M3 codes with a zero mantissa and
// exponent field e in 1..15 (2^-6 .. 2^8).  Then a s_a b s_b = (a b) 2^(ea +
// eb), so the packed codes go to the scaled FP4 MFMA (v_mfma_scale_f32_
// 32x32x64_f8f6f4) undecoded, with the scales as E8M0 exponents (e + 120).
// That MFMA applies one scale per lane to 32 K slots; NVFP4 scales cover 16,
// so each lane's 32 slots hold one 16-value block and 16 zeros: a step of
// four lanes-halves covers blocks 2 s (lanes 0-31) and 2 s + 1 (lanes 32-63)
// of every row, 32 real K per 32x32 MFMA (the fp16 path needs two MFMAs and
// eight decode instructions per fragment for the same 32 K).  Other scale
// codes are outside this path's contract (their mantissa bits are ignored).
//
// kScales, how the scales reach LDS.  kScalesPlain: [rows][K/16] scales, four
// 4-byte loads per lane per operand and K tile (8 bytes from each of 32 rows
// per instruction).  kScalesPairs (every K % 256 == 0): [rows][K/16] scales of
// two K tiles at once, one 16-byte load per lane and 64 rows (a row's 8 + 8
// bytes are adjacent), into one of two pair buffers (rows of 16 bytes; tile
// kt's 8 bytes at 8 (kt % 2)), half the instructions and half the cache lines
// per K tile.  The pair buffers reuse the stages' scale areas plus 4 KiB.
// kScalesBlocked: SFA and SFB arrive in the blocked layout the pages' kernels
// consume (512-byte atoms of 128 rows x 4 scale blocks, atoms of a 128-row
// tile in K order; row r, block c of an atom at (r % 32) * 16 + (r / 32) * 4 +
// c).  A 128 x 128 tile's scales for one 128-K tile are then its two
// consecutive atoms, 1 KiB, one 16-byte direct load per lane per operand,
// kept in LDS as they are; the compute reads row 32 i + l32's four blocks of
// 64-K group g at 512 g + 16 l32 + 4 i.  Rows past M or N are the layout's
// zero padding.
typedef __attribute__((address_space(3))) void lds_void;
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kScalesPlain = 0, kScalesPairs = 1, kScalesBlocked = 2;

// The 16 MFMAs of one power-of-two step: the scale bytes sit in byte kSel of
// each lane's exponent dwords.
template <int kSel>
__device__ inline void mfma_pow2_step(f32x16 (&acc)[4][4], const i32x8 (&fa)[4], const i32x8 (&fb)[4],
                                      const uint32_t (&ea)[4], const uint32_t (&eb)[4])
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa[i], fb[j], acc[i][j], 4, 4, kSel,
                                                                         (int)ea[i], kSel, (int)eb[j]);
}

// The work of one workgroup (one 128 x 128 tile); Table is the by-value
// GroupTable of an ordinary launch or a DevTableView of a device-resident one.
//
// kWaves = 4: four waves share the tile, each running the pipeline above over
// a quarter of its K tiles (whole pairs of K tiles with paired scales) in an
// LDS region of its own (the four regions fill the CU's 160 KiB), with no
// barrier in the K loop.  Their partial tiles are then added through LDS in a
// fixed order, (w0 + w2) + (w1 + w3), and wave 0 writes C.  One workgroup per
// CU: used where tiles are too few for one wave per tile to fill the SIMDs.
template <bool kPow2, int kScales, int kWaves, class Table>
__device__ inline void tiled_dma_tile(const Table &tab, const int w)
{
    constexpr bool kBlocked = kScales == kScalesBlocked;
    constexpr bool kPairs = kScales == kScalesPairs;
    static_assert(!kPow2 || kScales == kScalesPlain, "the power-of-two path reads plain scales");
    static_assert(kWaves == 1 || (!kPow2 && !kBlocked), "four-wave tiles read plain scales");
    using namespace tiled;
    constexpr int kWaveLds = 2 * kStageBytes + (kPairs ? 4096 : 0);
    static_assert(kWaves * kWaveLds <= 160 * 1024, "the wave regions fit in LDS");
    __shared__ __attribute__((aligned(16))) uint8_t stages_all[kWaves * kWaveLds];
    const int wv = kWaves > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
    uint8_t *const stages = kWaves == 1 ? stages_all : stages_all + wv * kWaveLds;
    uint8_t *const stage0 = stages;
    uint8_t *const stage1 = stages + kStageBytes;
    // pair buffers (kPairs): A's in the stages' 2 KiB scale areas, B's past them
    auto qa = [&](int q) { return stages + q * kStageBytes + kSaOff; };
    auto qb = [&](int q) { return stages + 2 * kStageBytes + 2048 * q; };

    const int gi = find_group(tab, w);
    const GemmDesc &d = tab.g[gi];
    const int r = w - tab.prefix[gi];
    const int tm = r % d.tiles_m;
    const int tn = r / d.tiles_m;
    const int M = d.M, N = d.N, K = d.K;
    const int row0 = tm * BM, col0 = tn * BN;
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const uint32_t sh = h * 16;

    const int kb_row = K / 2;
    const int ks_row = K / 16;
    const int nkt = K / BK;
    // this wave's K tiles [kt_lo, kt_hi): all of them, or a quarter (whole
    // pairs of K tiles when the scales move in pairs)
    const int kt_lo = kWaves == 1 ? 0 : kPairs ? 2 * ((nkt / 2) * wv / kWaves) : nkt * wv / kWaves;
    const int kt_hi = kWaves == 1 ? nkt : kPairs ? 2 * ((nkt / 2) * (wv + 1) / kWaves) : nkt * (wv + 1) / kWaves;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(d.A + (long)row0 * kb_row, (uint64_t)(M - row0) * kb_row);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(d.B + (long)col0 * kb_row, (uint64_t)(N - col0) * kb_row);
    // blocked scales: one 128-row tile's atoms, K / 64 of them (K % 128 == 0)
    const long atoms_bytes = (long)(K / 64) * 512;
    const __amdgpu_buffer_rsrc_t rSA =
        kBlocked ? make_rsrc(d.SFA + (long)tm * atoms_bytes, (uint64_t)atoms_bytes)
                 : make_rsrc(d.SFA + (long)row0 * ks_row, (uint64_t)(M - row0) * ks_row);
    const __amdgpu_buffer_rsrc_t rSB =
        kBlocked ? make_rsrc(d.SFB + (long)tn * atoms_bytes, (uint64_t)atoms_bytes)
                 : make_rsrc(d.SFB + (long)col0 * ks_row, (uint64_t)(N - col0) * ks_row);

    // data: instruction j covers rows 16 j .. 16 j + 15
    const int drow = lane >> 2;
    const uint32_t d_off = (uint32_t)(drow * kb_row + (((lane & 3) ^ ((drow >> 2) & 3)) << 4));
    // scales: instruction j covers rows 32 j .. 32 j + 31 (two dwords each)
    const uint32_t s_off = (uint32_t)((lane >> 1) * ks_row + (lane & 1) * 4);

    // tile kt into stage `st` (tiles past kt_hi read as zero)
    auto issue = [&](uint8_t *st, int kt) {
        const bool live = kt < kt_hi;
        const uint32_t kb = (uint32_t)kt * kRowBytes, ks = (uint32_t)kt * kSfBytes;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t off = live ? d_off + (uint32_t)(16 * j * kb_row) + kb : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_void *)(st + kAOff + 1024 * j), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_void *)(st + kBOff + 1024 * j), 16, off, 0, 0, 0);
        }
        if (kPairs) {
            // scales move in pairs of K tiles (issue_pair)
        } else if (kBlocked) {
            // the tile's two atoms of this K tile: 1 KiB per operand
            const uint32_t off = live ? (uint32_t)kt * 1024 + (uint32_t)(lane * 16) : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, (lds_void *)(st + kSaOff), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rSB, (lds_void *)(st + kSbOff), 16, off, 0, 0, 0);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t off = live ? s_off + (uint32_t)(32 * j * ks_row) + ks : kOutOfRange;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, (lds_void *)(st + kSaOff + 256 * j), 4, off, 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rSB, (lds_void *)(st + kSbOff + 256 * j), 4, off, 0, 0, 0);
            }
        }
    };
    // scales of K tiles kt and kt + 1 (kt even) into pair buffer q: instruction
    // j covers rows 64 j .. 64 j + 63, lane i row 64 j + i
    auto issue_pair = [&](int q, int kt) {
        const bool live = kt < kt_hi;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t off = live ? (uint32_t)((64 * j + lane) * ks_row + kt * kSfBytes) : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, (lds_void *)(qa(q) + 1024 * j), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rSB, (lds_void *)(qb(q) + 1024 * j), 16, off, 0, 0, 0);
        }
    };


    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (f32x16){};

    // MFMA work of the 128-K tile in stage st: two 64-K groups g.  Issue
    // order (scheduling groups): the LDS reads, the scale conversion and
    // first decode step, then every MFMA followed by the next step's decode
    // VALU (4 per MFMA, 5 across the group boundary, where the second
    // group's scales and first step are decoded), then the last step's MFMAs.
    // (kPairs: the scales come from pair buffer q, tile half `half`)
    auto compute = [&](const uint8_t *st, int q, int half) {
        half2_t ca[2][4], cb[2][4];
        u32x4 pa[2][4], pb[2][4];
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (kPairs) {
                    const int o = (32 * i + l32) * 16 + 8 * half + 4 * g;
                    const uint32_t wa = *(const uint32_t *)(qa(q) + o);
                    const uint32_t wb = *(const uint32_t *)(qb(q) + o);
                    ca[g][i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wa >> sh, 1.0f, false);
                    cb[g][i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb >> sh, 1.0f, false);
                } else if constexpr (kBlocked) {
                    // blocks 4 g .. 4 g + 3 of row 32 i + l32: word i of the row's 16 bytes in atom g
                    const uint32_t wa = *(const uint32_t *)(st + kSaOff + 512 * g + 16 * l32 + 4 * i);
                    const uint32_t wb = *(const uint32_t *)(st + kSbOff + 512 * g + 16 * l32 + 4 * i);
                    ca[g][i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wa >> sh, 1.0f, false);
                    cb[g][i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb >> sh, 1.0f, false);
                } else {
                    const u32x2 va = *(const u32x2 *)(st + kSaOff + (32 * i + l32) * kSfBytes);
                    const u32x2 vb = *(const u32x2 *)(st + kSbOff + (32 * i + l32) * kSfBytes);
                    ca[g][i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((g ? va.y : va.x) >> sh, 1.0f, false);
                    cb[g][i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((g ? vb.y : vb.x) >> sh, 1.0f, false);
                }
                pa[g][i] = *(const u32x4 *)(st + kAOff + swz(32 * i + l32, 2 * g + h));
                pb[g][i] = *(const u32x4 *)(st + kBOff + swz(32 * i + l32, 2 * g + h));
            }
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                half8_t fa[4], fb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    fa[i] = decode8(pa[g][i][q], q < 2 ? bcast_lo(ca[g][i]) : bcast_hi(ca[g][i]));
                    fb[i] = decode8(pb[g][i][q], q < 2 ? bcast_lo(cb[g][i]) : bcast_hi(cb[g][i]));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
        __builtin_amdgcn_sched_group_barrier(0x100, 32, 0); // LDS reads
        __builtin_amdgcn_sched_group_barrier(0x002, 80, 0); // group 0 scales + step 0 decode
#pragma unroll
        for (int k = 0; k < 48; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
#pragma unroll
        for (int k = 0; k < 16; ++k) { // group 1 scales + step 0 under group 0's last MFMAs
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
        }
#pragma unroll
        for (int k = 0; k < 48; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    };

    // power-of-two scales: step s (blocks 2 s + h of every row) of the 128-K
    // tile in stage st on the scaled FP4 MFMA
    auto compute_pow2 = [&](const uint8_t *st) {
        // E8M0 exponents of the lane's rows: dword d holds blocks 4 d + h ..
        // (shifted down by h bytes), so block 2 s + h sits in byte 2 (s % 2)
        // of dword s / 2
        uint32_t ea[2][4], eb[2][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x2 va = *(const u32x2 *)(st + kSaOff + (32 * i + l32) * kSfBytes);
            const u32x2 vb = *(const u32x2 *)(st + kSbOff + (32 * i + l32) * kSfBytes);
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                ea[d][i] = ((va[d] >> (8 * h + 3)) & 0x0F0F0F0Fu) + 0x78787878u;
                eb[d][i] = ((vb[d] >> (8 * h + 3)) & 0x0F0F0F0Fu) + 0x78787878u;
            }
        }
#pragma unroll
        for (int st4 = 0; st4 < 4; ++st4) {
            i32x8 fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const u32x2 xa = *(const u32x2 *)(st + kAOff + swz(32 * i + l32, st4) + 8 * h);
                const u32x2 xb = *(const u32x2 *)(st + kBOff + swz(32 * i + l32, st4) + 8 * h);
                fa[i] = (i32x8){(int)xa.x, (int)xa.y, 0, 0, 0, 0, 0, 0};
                fb[i] = (i32x8){(int)xb.x, (int)xb.y, 0, 0, 0, 0, 0, 0};
            }
            if (st4 & 1)
                mfma_pow2_step<2>(acc, fa, fb, ea[st4 >> 1], eb[st4 >> 1]);
            else
                mfma_pow2_step<0>(acc, fa, fb, ea[st4 >> 1], eb[st4 >> 1]);
        }
    };

    // The compiler does not order these loads' LDS writes before the reads
    // of the same array, so the waits are explicit: before a stage is read,
    // at most the other stage's kIssued loads may still be in flight
    // (s_waitcnt simm16 on gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4 and
    // lgkmcnt 11:8 left at their maxima).
    constexpr int kIssued = 8 + 8 + (kPairs ? 4 : kBlocked ? 2 : 8);
    constexpr int kWaitOther = ((kIssued >> 4) << 14) | (15 << 8) | (7 << 4) | (kIssued & 15);
    if (kPairs && kt_hi > kt_lo) {
        // stage data as below; scale pairs one iteration ahead.  Before each
        // compute, this iteration's data (16) and next pair (4), or next data
        // stage, may still be in flight: every wait leaves kIssued.
        issue(stage0, kt_lo);
        issue_pair(0, kt_lo);
        for (int kt = kt_lo, q = 0; kt < kt_hi; kt += 2, q ^= 1) {
            issue(stage1, kt + 1);
            issue_pair(q ^ 1, kt + 2);
            SCHED_FENCE();
            __builtin_amdgcn_s_waitcnt(kWaitOther); // stage0 and pair q have landed
            SCHED_FENCE();
            compute(stage0, q, 0);
            SCHED_FENCE();
            issue(stage0, kt + 2);
            SCHED_FENCE();
            __builtin_amdgcn_s_waitcnt(kWaitOther); // stage1 has landed
            SCHED_FENCE();
            compute(stage1, q, 1);
            SCHED_FENCE();
        }
    } else if (kt_hi > kt_lo) {
        issue(stage0, kt_lo);
        for (int kt = kt_lo; kt < kt_hi; kt += 2) {
            issue(stage1, kt + 1);
            SCHED_FENCE();
            __builtin_amdgcn_s_waitcnt(kWaitOther); // stage0 has landed
            SCHED_FENCE();
            if (kPow2)
                compute_pow2(stage0);
            else
                compute(stage0, 0, 0);
            SCHED_FENCE();
            issue(stage0, kt + 2);
            SCHED_FENCE();
            __builtin_amdgcn_s_waitcnt(kWaitOther); // stage1 has landed
            SCHED_FENCE();
            // with an odd tile count the last stage1 tile is out of range:
            // zeros, adding exact zeros (no branch around the accumulators)
            if (kPow2)
                compute_pow2(stage1);
            else
                compute(stage1, 0, 0);
            SCHED_FENCE();
        }
    }

    if constexpr (kWaves > 1) {
        // add the four partial tiles: 16-byte pieces (i, j, e / 4) of each
        // lane, [piece][lane], in slots of 64 KiB over the whole LDS
        __builtin_amdgcn_s_waitcnt(0); // this wave's trailing zero loads have landed
        __syncthreads();               // every wave is past its K loop
        float *red = (float *)stages_all;
        auto put = [&](int slot) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        *(float4 *)(red + slot * 16384 + (((i * 4 + j) * 4 + e) * 64 + lane) * 4) =
                            (float4){acc[i][j][4 * e], acc[i][j][4 * e + 1], acc[i][j][4 * e + 2], acc[i][j][4 * e + 3]};
        };
        auto add = [&](int slot) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float4 v = *(const float4 *)(red + slot * 16384 + (((i * 4 + j) * 4 + e) * 64 + lane) * 4);
                        acc[i][j][4 * e] += v.x;
                        acc[i][j][4 * e + 1] += v.y;
                        acc[i][j][4 * e + 2] += v.z;
                        acc[i][j][4 * e + 3] += v.w;
                    }
        };
        if (wv >= 2)
            put(wv - 2);
        __syncthreads();
        if (wv < 2)
            add(wv);
        __syncthreads();
        if (wv == 1)
            put(0);
        __syncthreads();
        if (wv != 0)
            return;
        add(0);
    }

    // epilogue: fp16 (round to nearest even) rows 0..63 into stage0 and rows
    // 64..127 into stage1 (the loop's last reads are done: each wave reads
    // only what it wrote), then 16-byte row-contiguous stores masked to M x N
    // (the tile's trailing zero-tile loads were out of range: nothing lands)
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * i + (e >> 2) * 8 + h * 4 + (e & 3);
                const int col = 32 * j + l32;
                uint8_t *sC = row < 64 ? stage0 : stage1;
                *(uint16_t *)(sC + (row & 63) * kCStride + col * 2) = __builtin_bit_cast(uint16_t, (_Float16)acc[i][j][e]);
            }
    const bool vec_ok = (N % 8 == 0) && ((((uintptr_t)d.C) & 15) == 0);
#pragma unroll 4
    for (int s2 = 0; s2 < BM * BN / 8 / 64; ++s2) {
        const int seg = s2 * 64 + lane;
        const int row = seg >> 4, c8 = (seg & 15) * 8;
        const int grow = row0 + row, gcol = col0 + c8;
        if (grow >= M)
            continue;
        const uint8_t *sC = row < 64 ? stage0 : stage1;
        uint16_t *dst = d.C + (long)grow * N + gcol;
        const uint16_t *src = (const uint16_t *)(sC + (row & 63) * kCStride + c8 * 2);
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

template <bool kPow2, int kScales>
__global__ __launch_bounds__(64) void gemm_tiled_dma_kernel(GroupTable tab)
{
    tiled_dma_tile<kPow2, kScales, 1>(tab, (int)blockIdx.x);
}

// Four waves per 128 x 128 tile, each over a quarter of its K.
template <int kScales>
__global__ __launch_bounds__(256) void gemm_tiled_dma4_kernel(GroupTable tab)
{
    tiled_dma_tile<false, kScales, 4>(tab, (int)blockIdx.x);
}

} // namespace
} // namespace nvfp4
