// kernels_wide.hip -- the 128 x 256 "wide" tile: four waves share decoded A
// fragments through LDS.
//
// The scale mapping and the MFMA operand placement are those of
// kernel_common.h: each nibble and its block scale are decoded to exact fp16
// values and fed to v_mfma_f32_32x32x16_f16 with fp32 accumulation.  Decode
// VALU work per MFMA sets the speed of that mapping, so this tile spreads the
// decode over the workgroup instead of repeating it in every wave:
//
//   * wave w owns output columns [64 w, 64 w + 64) of the tile for all 128
//     rows (4 x 2 MFMA blocks, 128 fp32 accumulators);
//   * wave w decodes its own 64 rows of B (used by no other wave) and A rows
//     [32 w, 32 w + 32), the row block it shares with the other three waves:
//     it keeps those fragments in registers and writes them to an LDS exchange
//     buffer, from which the other waves read them;
//   * per 16 K a wave decodes 3 fragments (24 VALU) for 8 MFMAs, where a wave
//     decoding all its own operands for the same 8 MFMAs would decode 6.
//
// Each wave moves only the raw rows it decodes (its 32 A rows and 64 B rows,
// plus their scales) from global memory straight into its own LDS region
// (buffer_load ... lds), two K tiles of 128 deep, so raw data needs no
// workgroup barrier.  The decoded fragments are exchanged one sub-step (32 K,
// two MFMA steps) ahead through two exchange buffers, with one LDS-only
// barrier per sub-step.  80 KiB of LDS and at most 256 registers per lane let
// two workgroups share a CU (two waves per SIMD).
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
constexpr int BM = 128, BN = 256, BK = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kARows = BM / kWaves;                        // 32: the wave's shared A row block
constexpr int kBRows = BN / kWaves;                        // 64: the wave's own B rows
constexpr int kRowBytes = BK / 2;                          // 64 packed bytes per row per K tile
constexpr int kAOff = 0;                                   // in a stage
constexpr int kBOff = kARows * kRowBytes;                  // 2048
constexpr int kStageBytes = (kARows + kBRows) * kRowBytes; // 6144
// scale pairs (two K tiles, 16 bytes per row): A rows in slots 0..31 of 64,
// B rows 0..63
constexpr int kPairA = 0, kPairB = 1024, kPairBytes = 2048;
constexpr int kWaveBytes = 2 * kStageBytes + 2 * kPairBytes; // 16384
constexpr int kXStep = 64 * 16;                              // one decoded fragment, 16 bytes per lane
constexpr int kXWave = 2 * kXStep;                           // two MFMA steps per sub-step
constexpr int kXBuf = kWaves * kXWave;
constexpr int kXOff = kWaves * kWaveBytes;
constexpr int kLdsBytes = kXOff + 2 * kXBuf; // 80 KiB
constexpr int kCStride = BN * 2 + 16;        // bytes per fp16 C row staged in LDS
static_assert(BM * kCStride <= kLdsBytes, "the C tile reuses the LDS");
static_assert(2 * kLdsBytes <= 160 * 1024, "two workgroups per CU");
// loads per K tile: A 2 and B 4 instructions, plus 2 for the scale pair on
// even tiles
constexpr int kLoadsOdd = 6, kLoadsEven = 8;
} // namespace wide

typedef __attribute__((address_space(3))) void wide_lds_void;

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

__device__ inline void wide_tile(const WideTable &tab, const int wid, uint8_t *ws)
{
    using namespace wide;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kLdsBytes];

    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
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
    // this slice's K tiles [kt_lo, nkt): whole pairs of K tiles
    const int npairs = K / (2 * BK);
    const int kt_lo = 2 * (int)((long)slice * npairs / S);
    const int nkt = 2 * (int)((long)(slice + 1) * npairs / S);

    // this wave's rows: A [arow, arow + 32), B [brow, brow + 64)
    const int arow = row0 + kARows * wv, brow = col0 + kBRows * wv;
    const int a_rows = max(0, min(kARows, M - arow)), b_rows = max(0, min(kBRows, N - brow));
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(d.A + (long)arow * kb_row, (uint64_t)a_rows * kb_row);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(d.B + (long)brow * kb_row, (uint64_t)b_rows * kb_row);
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(d.SFA + (long)arow * ks_row, (uint64_t)a_rows * ks_row);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(d.SFB + (long)brow * ks_row, (uint64_t)b_rows * ks_row);

    uint8_t *const region = lds + wv * kWaveBytes;
    uint8_t *const xbase = lds + kXOff;

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
        for (int j = 0; j < 2; ++j)
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
            const uint32_t ks = (uint32_t)kt * 8;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rSA, (wide_lds_void *)(pb + kPairA), 16,
                                                     live && lane < kARows ? pa_off + ks : kOutOfRange, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rSB, (wide_lds_void *)(pb + kPairB), 16,
                                                     live ? pa_off + ks : kOutOfRange, 0, 0, 0);
        }
    };

    // raw operands of one 64-K group: this lane's 16 packed bytes of its A row
    // and of its two B rows, and their scale words (blocks 4 g .. 4 g + 3,
    // shifted to this lane's half)
    u32x4 ra, rb0, rb1;
    uint32_t wa, wb0, wb1;
    auto read_raw = [&](int kt, int g) {
        const uint8_t *sb = region + (kt & 1) * kStageBytes;
        ra = *(const u32x4 *)(sb + kAOff + tiled::swz(l32, 2 * g + h));
        rb0 = *(const u32x4 *)(sb + kBOff + tiled::swz(l32, 2 * g + h));
        rb1 = *(const u32x4 *)(sb + kBOff + tiled::swz(32 + l32, 2 * g + h));
        const uint8_t *pb = region + 2 * kStageBytes + ((kt >> 1) & 1) * kPairBytes + 8 * (kt & 1) + 4 * g;
        wa = *(const uint32_t *)(pb + kPairA + 16 * l32) >> sh;
        wb0 = *(const uint32_t *)(pb + kPairB + 16 * l32) >> sh;
        wb1 = *(const uint32_t *)(pb + kPairB + 16 * (32 + l32)) >> sh;
    };

    // fragments of the current sub-step (A_cur: this wave's row block) and of
    // the next (decoded during the current one)
    half8_t A_cur[2], B_cur[2][2], A_nx[2], B_nx[2][2];
    // decode this lane's fragments of half `qq` of the group in ra/rb
    auto decode = [&](int qq) {
        const half2_t ca = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wa, 1.0f, false);
        const half2_t cb0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb0, 1.0f, false);
        const half2_t cb1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(wb1, 1.0f, false);
        const half2_t sa = qq ? bcast_hi(ca) : bcast_lo(ca);
        const half2_t sb0 = qq ? bcast_hi(cb0) : bcast_lo(cb0);
        const half2_t sb1 = qq ? bcast_hi(cb1) : bcast_lo(cb1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            A_nx[s] = decode8(ra[2 * qq + s], sa);
            B_nx[0][s] = decode8(rb0[2 * qq + s], sb0);
            B_nx[1][s] = decode8(rb1[2 * qq + s], sb1);
        }
    };
    auto put_x = [&](int buf) {
#pragma unroll
        for (int s = 0; s < 2; ++s)
            *(half8_t *)(xbase + buf * kXBuf + wv * kXWave + s * kXStep + lane * 16) = A_nx[s];
    };

    // accumulators: acc[t][f] is row block (wv + t) % 4, column block f of
    // this wave's 64 columns
    f32x16 acc[4][2];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int f = 0; f < 2; ++f)
            acc[t][f] = (f32x16){};

    // one sub-step (32 K): the other waves' row blocks from exchange buffer
    // xb (read_x), then the raw read and decode of the next sub-step, 16
    // MFMAs, and the next fragments into the other exchange buffer
    half8_t Ao[3][2];
    auto read_x = [&](int xb) {
#pragma unroll
        for (int t = 1; t < 4; ++t)
#pragma unroll
            for (int s = 0; s < 2; ++s)
                Ao[t - 1][s] = *(const half8_t *)(xbase + xb * kXBuf + ((wv + t) & 3) * kXWave + s * kXStep + lane * 16);
    };
    auto mfmas = [&]() {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
#pragma unroll
            for (int f = 0; f < 2; ++f)
                acc[0][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A_cur[s], B_cur[f][s], acc[0][f], 0, 0, 0);
#pragma unroll
            for (int t = 1; t < 4; ++t)
#pragma unroll
                for (int f = 0; f < 2; ++f)
                    acc[t][f] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Ao[t - 1][s], B_cur[f][s], acc[t][f], 0, 0, 0);
        }
    };
    auto advance = [&]() {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            A_cur[s] = A_nx[s];
            B_cur[0][s] = B_nx[0][s];
            B_cur[1][s] = B_nx[1][s];
        }
    };

    // prologue: the slice's first two K tiles in flight, the first landed, its
    // sub-step 0 decoded and exchanged
    issue(0, kt_lo, true);
    issue(1, kt_lo + 1, false);
    WAIT_VM(kLoadsOdd);
    read_raw(kt_lo, 0);
    decode(0);
    put_x(0);
    advance();
    LDS_BARRIER();

    // sub-step u of K tile kt (u = 0..3; kPar = kt % 2), exchange buffer u % 2
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
        LDS_BARRIER();                                                                                               \
    } while (0)

    for (int kt = kt_lo; kt < nkt; kt += 2) {
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

    // the trailing (out-of-range) loads have landed and every wave is past its
    // last LDS access
    __builtin_amdgcn_s_waitcnt(0);
    LDS_BARRIER();

    if (S > 1) {
        // partial tile of this slice: float4 q (0..31) of thread t at
        // (q * 256 + t) * 16 bytes of its slot, so each store is contiguous
        float *const parts = (float *)(ws + kCounterBytes);
        const long tile_slot0 = (long)d.slot0 + (long)tile_local * S;
        const int tid = (int)threadIdx.x;
        float4 *mine = (float4 *)(parts + (tile_slot0 + slice) * (BM * BN));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4)
                    mine[((t * 2 + f) * 4 + e4) * kThreads + tid] =
                        (float4){acc[t][f][4 * e4], acc[t][f][4 * e4 + 1], acc[t][f][4 * e4 + 2], acc[t][f][4 * e4 + 3]};
        int *const counter = (int *)ws + d.cnt0 + tile_local;
        __syncthreads(); // every thread's partial stores precede the ticket
        if (tid == 0) {
            const bool last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
            if (last)
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            *(volatile int *)lds = last ? 1 : 0;
        }
        __syncthreads();
        const bool last = *(volatile int *)lds != 0;
        __syncthreads(); // the flag is read before the C tile reuses the LDS
        if (!last)
            return;
        // the slices in slice order
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const int q = (t * 2 + f) * 4 + e4;
                    float4 sum = (float4){0.f, 0.f, 0.f, 0.f};
                    for (int j = 0; j < S; ++j) {
                        const float4 v = j == slice ? (float4){acc[t][f][4 * e4], acc[t][f][4 * e4 + 1],
                                                                acc[t][f][4 * e4 + 2], acc[t][f][4 * e4 + 3]}
                                                    : ((const float4 *)(parts + (tile_slot0 + j) * (BM * BN)))[q * kThreads + tid];
                        if (j == 0)
                            sum = v;
                        else
                            sum += v;
                    }
                    acc[t][f][4 * e4] = sum.x;
                    acc[t][f][4 * e4 + 1] = sum.y;
                    acc[t][f][4 * e4 + 2] = sum.z;
                    acc[t][f][4 * e4 + 3] = sum.w;
                }
        if (tid == 0)
            __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); // for the next launch
    }

    // epilogue: fp16 (round to nearest even) into an LDS C tile, then 16-byte
    // row-contiguous stores masked to M x N
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int i = (wv + t) & 3;
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * i + (e >> 2) * 8 + h * 4 + (e & 3);
                const int col = 64 * wv + 32 * f + l32;
                *(uint16_t *)(lds + row * kCStride + col * 2) = __builtin_bit_cast(uint16_t, (_Float16)acc[t][f][e]);
            }
    }
    LDS_BARRIER();
    const bool vec_ok = (N % 8 == 0) && ((((uintptr_t)d.C) & 15) == 0);
#pragma unroll 4
    for (int s2 = 0; s2 < BM * BN / 8 / kThreads; ++s2) {
        const int seg = s2 * kThreads + (int)threadIdx.x;
        const int row = seg >> 5, c8 = (seg & 31) * 8;
        const int grow = row0 + row, gcol = col0 + c8;
        if (grow >= M || gcol >= N)
            continue;
        uint16_t *dst = d.C + (long)grow * N + gcol;
        const uint16_t *src = (const uint16_t *)(lds + row * kCStride + c8 * 2);
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

__global__ __launch_bounds__(wide::kThreads, 2) void gemm_wide_kernel(WideTable tab, uint8_t *ws)
{
    wide_tile(tab, (int)blockIdx.x, ws);
}

} // namespace

hipError_t launch_wide(const WideTable &table, void *workspace, hipStream_t stream)
{
    const int wgs = table.prefix[table.num_groups];
    if (wgs <= 0)
        return hipSuccess;
    for (int g = 0; g < table.num_groups; ++g) {
        const WideDesc &d = table.g[g];
        const int n = (table.prefix[g + 1] - table.prefix[g]) / max(1, d.split);
        if (d.K % (2 * wide::BK) != 0 || ((((uintptr_t)d.SFA) | ((uintptr_t)d.SFB)) & 15) != 0 ||
            ((((uintptr_t)d.A) | ((uintptr_t)d.B)) & 15) != 0 || d.tiles_m != (d.M + wide::BM - 1) / wide::BM ||
            d.tiles_n != (d.N + wide::BN - 1) / wide::BN || d.split < 1 ||
            n * d.split != table.prefix[g + 1] - table.prefix[g] || d.tile0 < 0 ||
            (long long)d.tile0 + n > (long long)d.tiles_m * d.tiles_n ||
            (d.split > 1 && (workspace == nullptr || d.split > d.K / (2 * wide::BK) || d.cnt0 < 0 ||
                             d.cnt0 + n > kMaxSplitTiles || d.slot0 < 0)))
            return hipErrorInvalidValue;
    }
    uint8_t *ws = (uint8_t *)workspace;
    void *args[] = {const_cast<WideTable *>(&table), &ws};
    return hipLaunchKernel((const void *)gemm_wide_kernel, dim3((unsigned)wgs), dim3(wide::kThreads), args, 0,
                           stream);
}

} // namespace nvfp4
