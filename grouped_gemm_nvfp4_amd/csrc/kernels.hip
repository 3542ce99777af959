// kernels.hip -- gfx950 (CDNA4) kernels for NVFP4 block-scaled GEMM.
//
// C[m][n] = fp16_rne( sum_k (A[m][k] * SFA[m][k/16]) * (B[n][k] * SFB[n][k/16]) )
// (kernelbot pages nvfp4-group-gemm-498453 / nvfp4-gemm-125598, block-scaled MMA
// loop; raw-CUDA page nvfp4-group-gemm-407526, round-to-nearest fp16 epilogue).
//
// Scale mapping onto CDNA4.  gfx950's scaled FP4 matrix instructions take one
// power-of-two (e8m0) scale per 32 K elements, while NVFP4 carries a full e4m3
// scale (4 significant bits) per 16.  Every element times its scale,
// e2m1 * e4m3, has at most 6 significant bits and lies in [2^-10, 2688], so it
// is exact in binary16; the product of two such values is exact in fp32.  The
// kernels therefore decode each nibble to fp16 (v_cvt_scalef32_pk_f16_fp4 with
// unit scale), multiply by the block's scale decoded to fp16
// (v_cvt_scalef32_pk_f16_fp8, then v_pk_mul_f16: exact), and feed
// v_mfma_f32_32x32x16_f16 with fp32 accumulation.  Only the fp32 accumulation
// rounds.  The scaled FP4/FP8 matrix instructions cannot carry the e4m3
// mantissa without error, so they are not used.
//
// MFMA operand placement.  For v_mfma_f32_32x32x16_f16 lane l supplies 8 fp16
// of A row (l % 32) and 8 fp16 of B column (l % 32); both halves of the wave
// (l / 32) supply different K slots.  The sum over K does not care which K
// index sits in which slot as long as A and B agree, so each lane takes 16
// contiguous packed bytes (32 K elements) of its row per 64-K group: half 0
// takes K [0, 32) and half 1 takes K [32, 64) of the group, one dword (8 K)
// per instruction.  Every dword lies inside one 16-element scale block.
//
// Accumulator layout of v_mfma_f32_32x32x16_f16: lane l, register r holds
// row 8*(r/4) + 4*(l/32) + (r%4), column l % 32.
#include "launch.h"

namespace nvfp4 {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw (unstrided) buffer resource: loads at offsets >= num_records return 0.
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kOutOfRange = 0x80000000u;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint64_t bytes)
{
    int n = bytes >= 0x7fffffffull ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, kBufferWord3);
}

// 8 packed e2m1 codes -> 8 fp16 values times the broadcast scale s.
__device__ inline half8_t decode8(uint32_t packed, half2_t s)
{
    half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 0);
    half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 1);
    half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2);
    half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 3);
    h0 *= s;
    h1 *= s;
    h2 *= s;
    h3 *= s;
    return (half8_t){h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
}

__device__ inline half2_t bcast_lo(half2_t v) { return (half2_t){v.x, v.x}; }
__device__ inline half2_t bcast_hi(half2_t v) { return (half2_t){v.y, v.y}; }

// Workgroup -> (group, tile) through the exclusive prefix over tile counts.
__device__ inline int find_group(const GroupTable &t, int w)
{
    int lo = 0, hi = t.num_groups;
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (t.prefix[mid] <= w)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// Tiled kernel: one workgroup of 256 threads (4 waves, 2x2) per BM x BN output
// tile, K consumed in BK-element tiles staged through LDS, double-buffered.
// ---------------------------------------------------------------------------
template <int BM, int BN, int BK>
struct TiledCfg {
    static constexpr int kThreads = 256;
    static constexpr int kWavesM = 2, kWavesN = 2;
    static constexpr int kWaveM = BM / kWavesM, kWaveN = BN / kWavesN;
    static constexpr int kFragM = kWaveM / 32, kFragN = kWaveN / 32;
    static constexpr int kRowBytes = BK / 2;          // packed bytes per row per K tile
    static constexpr int kStride = kRowBytes + 16;    // padded LDS row (bank spread)
    static constexpr int kSfBytes = BK / 16;          // scale bytes per row per K tile
    static constexpr int kStageBytes = (BM + BN) * kStride + (BM + BN) * kSfBytes;
    static constexpr int kCStride = BN + 8;           // fp16 elements per LDS C row
    static constexpr int kSmemBytes =
        (2 * kStageBytes > BM * kCStride * 2) ? 2 * kStageBytes : BM * kCStride * 2;
    static_assert(BK == 128, "scale handling below assumes 8 scale bytes per row");
    static_assert(BM == 128 && BN == 128, "load distribution assumes 128x128");
};

template <int BM, int BN, int BK>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(GroupTable tab)
{
    using Cfg = TiledCfg<BM, BN, BK>;
    __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::kSmemBytes];

    const int w = blockIdx.x;
    const int gi = find_group(tab, w);
    const GemmDesc &d = tab.g[gi];
    const int r = w - tab.prefix[gi];
    const int tm = r % d.tiles_m;
    const int tn = r / d.tiles_m;
    const int M = d.M, N = d.N, K = d.K;
    const int row0 = tm * BM, col0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform
    const int wm = wave / Cfg::kWavesN, wn = wave % Cfg::kWavesN;
    const int half_id = lane >> 5; // which K half of the 64-K group
    const int l32 = lane & 31;

    const long kb_row = K / 2;   // packed bytes per row
    const long ks_row = K / 16;  // scale bytes per row
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(d.A + (long)row0 * kb_row, (uint64_t)(M - row0) * kb_row);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(d.B + (long)col0 * kb_row, (uint64_t)(N - col0) * kb_row);
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(d.SFA + (long)row0 * ks_row, (uint64_t)(M - row0) * ks_row);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(d.SFB + (long)col0 * ks_row, (uint64_t)(N - col0) * ks_row);

    const int nk = (K + BK - 1) / BK;
    const bool sf_vec_ok = (K % BK) == 0 &&
                           ((((uintptr_t)d.SFA) | ((uintptr_t)d.SFB)) & 7) == 0;

    // Per-thread global load slots: 2 A chunks, 2 B chunks (16 B each) and one
    // 8-byte scale row (threads 0..127: SFA rows, 128..255: SFB rows).
    u32x4 ga[2], gb[2];
    u32x2 gs;

    auto load_tile = [&](int kt) {
        const int kbyte0 = kt * Cfg::kRowBytes;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + i * 256;
            const int row = c >> 2, col = c & 3;
            const int kb = kbyte0 + col * 16;
            const uint32_t off = (kb < kb_row) ? (uint32_t)(row * kb_row + kb) : kOutOfRange;
            ga[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0);
            gb[i] = __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0);
        }
        const int srow = tid & 127;
        const __amdgpu_buffer_rsrc_t rs = (wave < 2) ? rSA : rSB; // waves 0-1: SFA rows
        const uint32_t sbase = (uint32_t)(srow * ks_row + kt * Cfg::kSfBytes);
        if (sf_vec_ok) {
            gs = __builtin_amdgcn_raw_buffer_load_b64(rs, sbase, 0, 0);
        } else {
            // tail or unaligned: byte loads, blocks past K read as 0
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const bool ok = (kt * Cfg::kSfBytes + b) < ks_row;
                const uint32_t v = __builtin_amdgcn_raw_buffer_load_b8(rs, ok ? sbase + b : kOutOfRange, 0, 0);
                if (b < 4)
                    lo |= v << (8 * b);
                else
                    hi |= v << (8 * (b - 4));
            }
            gs = (u32x2){lo, hi};
        }
    };

    auto store_tile = [&](int buf) {
        uint8_t *st = smem + buf * Cfg::kStageBytes;
        uint8_t *sA = st;
        uint8_t *sB = st + BM * Cfg::kStride;
        uint8_t *sS = st + (BM + BN) * Cfg::kStride; // SFA rows then SFB rows
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + i * 256;
            const int row = c >> 2, col = c & 3;
            *(u32x4 *)(sA + row * Cfg::kStride + col * 16) = ga[i];
            *(u32x4 *)(sB + row * Cfg::kStride + col * 16) = gb[i];
        }
        *(u32x2 *)(sS + tid * Cfg::kSfBytes) = gs;
    };

    f32x16 acc[Cfg::kFragM][Cfg::kFragN];
#pragma unroll
    for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::kFragN; ++j)
            acc[i][j] = (f32x16){};

    auto compute_tile = [&](int buf) {
        const uint8_t *st = smem + buf * Cfg::kStageBytes;
        const uint8_t *sA = st;
        const uint8_t *sB = st + BM * Cfg::kStride;
        const uint8_t *sSA = st + (BM + BN) * Cfg::kStride;
        const uint8_t *sSB = sSA + BM * Cfg::kSfBytes;

        // scales: for this lane's half, blocks {2h, 2h+1} of 64-K group 0 and
        // {4+2h, 5+2h} of group 1, as fp16 pairs
        half2_t sa[Cfg::kFragM][2], sb[Cfg::kFragN][2];
#pragma unroll
        for (int i = 0; i < Cfg::kFragM; ++i) {
            const u32x2 v = *(const u32x2 *)(sSA + (wm * Cfg::kWaveM + i * 32 + l32) * Cfg::kSfBytes);
            const uint32_t sel = half_id ? ((v.x >> 16) | (v.y & 0xffff0000u))
                                         : ((v.x & 0xffffu) | (v.y << 16));
            sa[i][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sel, 1.0f, false);
            sa[i][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sel, 1.0f, true);
        }
#pragma unroll
        for (int j = 0; j < Cfg::kFragN; ++j) {
            const u32x2 v = *(const u32x2 *)(sSB + (wn * Cfg::kWaveN + j * 32 + l32) * Cfg::kSfBytes);
            const uint32_t sel = half_id ? ((v.x >> 16) | (v.y & 0xffff0000u))
                                         : ((v.x & 0xffffu) | (v.y << 16));
            sb[j][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sel, 1.0f, false);
            sb[j][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sel, 1.0f, true);
        }

#pragma unroll
        for (int g = 0; g < BK / 64; ++g) {
            u32x4 pa[Cfg::kFragM], pb[Cfg::kFragN];
#pragma unroll
            for (int i = 0; i < Cfg::kFragM; ++i)
                pa[i] = *(const u32x4 *)(sA + (wm * Cfg::kWaveM + i * 32 + l32) * Cfg::kStride +
                                         g * 32 + half_id * 16);
#pragma unroll
            for (int j = 0; j < Cfg::kFragN; ++j)
                pb[j] = *(const u32x4 *)(sB + (wn * Cfg::kWaveN + j * 32 + l32) * Cfg::kStride +
                                         g * 32 + half_id * 16);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                half8_t fa[Cfg::kFragM], fb[Cfg::kFragN];
#pragma unroll
                for (int i = 0; i < Cfg::kFragM; ++i)
                    fa[i] = decode8(pa[i][q], (q < 2) ? bcast_lo(sa[i][g]) : bcast_hi(sa[i][g]));
#pragma unroll
                for (int j = 0; j < Cfg::kFragN; ++j)
                    fb[j] = decode8(pb[j][q], (q < 2) ? bcast_lo(sb[j][g]) : bcast_hi(sb[j][g]));
#pragma unroll
                for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
                    for (int j = 0; j < Cfg::kFragN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
            }
        }
    };

    if (nk > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk)
                load_tile(kt + 1);
            compute_tile(cur);
            if (kt + 1 < nk)
                store_tile(cur ^ 1);
            __syncthreads();
        }
    }

    // Epilogue: fp32 -> fp16 (round to nearest even) through LDS, then
    // row-contiguous stores masked to M x N.
    uint16_t *sC = (uint16_t *)smem;
#pragma unroll
    for (int i = 0; i < Cfg::kFragM; ++i)
#pragma unroll
        for (int j = 0; j < Cfg::kFragN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm * Cfg::kWaveM + i * 32 + (e >> 2) * 8 + half_id * 4 + (e & 3);
                const int col = wn * Cfg::kWaveN + j * 32 + l32;
                sC[row * Cfg::kCStride + col] = __builtin_bit_cast(uint16_t, (_Float16)acc[i][j][e]);
            }
    __syncthreads();

    const bool vec_ok = (N % 8 == 0) && ((((uintptr_t)d.C) & 15) == 0);
    constexpr int kSegsPerRow = BN / 8;
#pragma unroll
    for (int s = 0; s < (BM * kSegsPerRow) / 256; ++s) {
        const int seg = tid + s * 256;
        const int row = seg / kSegsPerRow;
        const int c8 = (seg % kSegsPerRow) * 8;
        const int grow = row0 + row, gcol = col0 + c8;
        if (grow >= M)
            continue;
        uint16_t *dst = d.C + (long)grow * N + gcol;
        const uint16_t *src = sC + row * Cfg::kCStride + c8;
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

// ---------------------------------------------------------------------------
// Skinny kernel for small M: one workgroup of 512 threads (8 waves) per
// 64 x 256 output tile and K slice.  Wave w owns output columns
// [64 (w%4), +64) over half of every K tile (64-K groups 2 (w/4) and
// 2 (w/4) + 1); the two K halves are added through LDS at the end.  A 64 x 64
// wave tile reads each A fragment from LDS once for two B column blocks: LDS
// bandwidth (about 180 B/clk/CU measured), not MFMA, bounds a 64 x 32 tile.
//
// Memory side.  Every K tile (256 elements) the workgroup needs 256 B rows x
// 128 packed bytes, their 16 scale bytes, and 64 A rows x 128 bytes.  Each
// load instruction reads whole 128-byte lines (a wave covers 8 rows x 8 x 16
// bytes), kDepth K tiles ahead, into registers; one step before use the
// registers go to a double-buffered LDS stage: B and its scales as they are
// (rows padded to 144 bytes so both the row-wise writes and the MFMA-layout
// reads are bank-conflict free), A decoded to fp16 (each A element decoded
// once per workgroup).
//
// Math side.  A wave reads, per 64-K group and B column block, 16 bytes of the
// lane's B row for its half of the group, decodes 8 elements per 16 K
// (v_cvt_scalef32_pk_f16_fp4 then v_pk_mul_f16 by the block scale) and runs
// four 32x32x16 MFMAs: A rows 0-31 and 32-63 against its two column blocks.
//
// The K loop is a software pipeline, one step per K tile: compute tile t from
// LDS stage t&1, refill register slot X with tile t + kDepth, move slot Y
// (tile t + 1) into stage (t+1)&1, barrier.  sched_barrier fences stop the
// compiler from hoisting the refill above the code that still reads the slot,
// so it counts outstanding loads exactly instead of draining them.
//
// With split_k > 1 the K tiles are divided among split_k workgroups per output
// tile and each writes its fp32 accumulators, in their MFMA register layout,
// to the workspace; reduce_partials_kernel adds them in slice order.
// ---------------------------------------------------------------------------
namespace skinny {
constexpr int BM = 64, BN = 256, BK = 256;
constexpr int kThreads = 512;
#ifndef NVFP4_SKINNY_DEPTH
#define NVFP4_SKINNY_DEPTH 2
#endif
constexpr int kDepth = NVFP4_SKINNY_DEPTH; // K tiles in flight per thread
constexpr int kA16Stride = BK * 2 + 16;    // bytes per decoded A row (padded)
constexpr int kBStride = BK / 2 + 16;      // bytes per packed B row (padded)
constexpr int kA16Bytes = BM * kA16Stride;
constexpr int kBBytes = BN * kBStride;
constexpr int kSfbBytes = BN * (BK / 16);
constexpr int kStageBytes = kA16Bytes + kBBytes + kSfbBytes;
constexpr int kTileElems = BM * BN;        // partial-sum floats per tile
static_assert(2 * kStageBytes <= 160 * 1024, "two stages must fit in LDS");
} // namespace skinny

struct SkinnySlot {
    u32x4 b[4];    // B chunks j = 0..3: row 64j + tid/8, bytes [16 (tid%8), +16)
    u32x4 sfb;     // threads 0..255: the 16 scale bytes of B row tid
    u32x4 a;       // A: row tid/8, 32 elements at K [32 (tid%8), +32)
    uint32_t sfa;  // their two scale bytes
};

#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

// kVec: K % 256 == 0 and SFB 16-byte aligned, so a row's 16 scale bytes of a
// K tile are one aligned load.  Otherwise they are 8 two-byte loads (K % 32
// == 0 makes each pair of blocks wholly inside or wholly past K) whose bytes
// past K read as zero.
template <bool kVec>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(GroupTable tab, float *partials)
{
    using namespace skinny;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kStageBytes];

    const int S = tab.split_k;
    const int tile = blockIdx.x / S;
    const int split = blockIdx.x - tile * S;
    const int gi = find_group(tab, tile);
    const GemmDesc &d = tab.g[gi];
    const int r = tile - tab.prefix[gi];
    const int tm = r % d.tiles_m;
    const int tn = r / d.tiles_m;
    const int M = d.M, N = d.N, K = d.K;
    const int row0 = tm * BM, col0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // wave-uniform
    const int h = lane >> 5;
    const int l32 = lane & 31;

    const int kb_row = K / 2;
    const int ks_row = K / 16;
    const int nkt = (K + BK - 1) / BK;
    const int kt0 = (int)((long)split * nkt / S);
    const int kt1 = (int)((long)(split + 1) * nkt / S);

    // this workgroup's B rows [col0, col0 + 256); rows past N read as zero
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(d.B + (long)col0 * kb_row, (uint64_t)(N - col0) * kb_row);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(d.SFB + (long)col0 * ks_row, (uint64_t)(N - col0) * ks_row);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(d.A + (long)row0 * kb_row, (uint64_t)(M - row0) * kb_row);
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(d.SFA + (long)row0 * ks_row, (uint64_t)(M - row0) * ks_row);

    // loop-invariant per-thread offsets
    const int crow = tid >> 3, c16 = tid & 7; // chunk row (within 64) and 16-byte column
    uint32_t boff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        boff[j] = (uint32_t)((64 * j + crow) * kb_row + c16 * 16);
    const uint32_t sboff = (uint32_t)((tid & 255) * ks_row);
    const uint32_t aoff = (uint32_t)(crow * kb_row + c16 * 16);
    const uint32_t saoff = (uint32_t)(crow * ks_row + c16 * 2);
    const bool sfb_loader = wave < 4; // waves 0-3 carry the B scales

    auto load = [&](SkinnySlot &s, int kt) {
        const bool live = kt < kt1;
        const uint32_t kb = (uint32_t)kt * (BK / 2), ks = (uint32_t)kt * (BK / 16);
        // a 16-byte chunk at column c16 holds K [kt*256 + 32 c16, +32): wholly
        // inside or wholly past K
        const bool cin = live && (int)(kb + c16 * 16) < kb_row;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s.b[j] = __builtin_amdgcn_raw_buffer_load_b128(rB, cin ? boff[j] + kb : kOutOfRange, 0, 0);
        if (sfb_loader) {
            if (kVec) {
                s.sfb = __builtin_amdgcn_raw_buffer_load_b128(rSB, live ? sboff + ks : kOutOfRange, 0, 0);
            } else {
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const bool ok0 = live && (int)(ks + 4 * p) < ks_row;
                    const bool ok1 = live && (int)(ks + 4 * p + 2) < ks_row;
                    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rSB, ok0 ? sboff + ks + 4 * p : kOutOfRange, 0, 0);
                    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rSB, ok1 ? sboff + ks + 4 * p + 2 : kOutOfRange, 0, 0);
                    s.sfb[p] = lo | (hi << 16);
                }
            }
        }
        s.a = __builtin_amdgcn_raw_buffer_load_b128(rA, cin ? aoff + kb : kOutOfRange, 0, 0);
        s.sfa = __builtin_amdgcn_raw_buffer_load_b16(rSA, cin ? saoff + ks : kOutOfRange, 0, 0);
    };

    // slot -> LDS stage, in two parts so they can sit between the two halves
    // of the previous tile's MFMA work: A decoded to fp16, then packed B and
    // its scales as they are
    auto stage_a = [&](const SkinnySlot &s, int buf) {
        uint8_t *st = lds + buf * kStageBytes;
        const half2_t sc = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(s.sfa, 1.0f, false);
        uint8_t *dst = st + crow * kA16Stride + c16 * 64;
        *(half8_t *)(dst + 0) = decode8(s.a.x, bcast_lo(sc));
        *(half8_t *)(dst + 16) = decode8(s.a.y, bcast_lo(sc));
        *(half8_t *)(dst + 32) = decode8(s.a.z, bcast_hi(sc));
        *(half8_t *)(dst + 48) = decode8(s.a.w, bcast_hi(sc));
    };
    auto stage_b = [&](const SkinnySlot &s, int buf) {
        uint8_t *sb = lds + buf * kStageBytes + kA16Bytes;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *(u32x4 *)(sb + (64 * j + crow) * kBStride + c16 * 16) = s.b[j];
        if (sfb_loader)
            *(u32x4 *)(sb + kBBytes + tid * 16) = s.sfb;
    };

    const int nq = wave & 3;  // 64-column block of this wave
    const int kh = wave >> 2; // K half of every K tile
    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
            acc[a][b] = (f32x16){};
    const uint32_t sh = h * 16;

    // MFMA work of one 64-K group (ii = 0, 1 of this wave's K half)
    auto compute = [&](int buf, int ii) {
        const uint8_t *st = lds + buf * kStageBytes;
        const uint8_t *arow0 = st + l32 * kA16Stride + h * 64;
        const uint8_t *arow1 = arow0 + 32 * kA16Stride;
        const uint8_t *bro[2];
        u32x4 sfrow[2];
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int brow = nq * 64 + c * 32 + l32;
            bro[c] = st + kA16Bytes + brow * kBStride + h * 16;
            sfrow[c] = *(const u32x4 *)(st + kA16Bytes + kBBytes + brow * 16);
        }
        {
            const int i = 2 * kh + ii; // 64-K group
            // issue every LDS read of the group before the first MFMA
            u32x4 bq[2];
            half8_t fa[4][2];
#pragma unroll
            for (int c = 0; c < 2; ++c)
                bq[c] = *(const u32x4 *)(bro[c] + i * 32);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                fa[q][0] = *(const half8_t *)(arow0 + i * 128 + q * 16);
                fa[q][1] = *(const half8_t *)(arow1 + i * 128 + q * 16);
            }
            half2_t sb[2];
#pragma unroll
            for (int c = 0; c < 2; ++c)
                // scales of this lane's half in group i: blocks 4i+2h, 4i+2h+1
                sb[c] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sfrow[c][i] >> sh, 1.0f, false);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const half8_t fb = decode8(bq[c][q], q < 2 ? bcast_lo(sb[c]) : bcast_hi(sb[c]));
                    acc[0][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[q][0], fb, acc[0][c], 0, 0, 0);
                    acc[1][c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[q][1], fb, acc[1][c], 0, 0, 0);
                }
            }
        }
    };

    // one pipeline step: refill slot X (staged into LDS last step) with tile
    // t + kDepth, run tile t's MFMA work from stage t&1 with slot Y (tile
    // t + 1) moved into stage (t+1)&1 between its two halves, barrier.  Steps
    // past the slice's last tile only keep the pipeline's shape: no MFMA
    // work, and their loads read zeros.
    auto step = [&](int t, SkinnySlot &X, SkinnySlot &Y) {
        load(X, t + kDepth);
        SCHED_FENCE();
        const bool live = t < kt1;
        if (live)
            compute(t & 1, 0);
        stage_a(Y, (t + 1) & 1);
        if (live)
            compute(t & 1, 1);
        stage_b(Y, (t + 1) & 1);
        __syncthreads();
        SCHED_FENCE();
    };

    if (kt1 > kt0) {
        SkinnySlot sl[kDepth]; // indexed by constants only: stays in registers
#pragma unroll
        for (int j = 0; j < kDepth; ++j) {
            load(sl[j], kt0 + j);
            SCHED_FENCE();
        }
        stage_a(sl[0], kt0 & 1);
        stage_b(sl[0], kt0 & 1);
        __syncthreads();
        SCHED_FENCE();
        // slot 0 is in LDS: the first step refills it
        for (int t = kt0; t < kt1; t += kDepth) {
#pragma unroll
            for (int j = 0; j < kDepth; ++j)
                step(t + j, sl[j], sl[(j + 1) % kDepth]);
        }
    }

    // add the two K halves: waves 4-7 hand their sums to waves 0-3 via LDS
    // (the stages are free: the loop ended with a barrier)
    float *red = (float *)lds + nq * (4 * 16 * 64) + lane;
    if (kh == 1) {
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    red[((a * 2 + b) * 16 + e) * 64] = acc[a][b][e];
    }
    __syncthreads();
    if (kh == 1)
        return;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[a][b][e] += red[((a * 2 + b) * 16 + e) * 64];

    if (S > 1) {
        // partial tile in register layout: [nq][rb][cb][reg][lane]
        float *dst = partials + ((long)tile * S + split) * kTileElems + nq * (4 * 16 * 64) + lane;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    dst[((a * 2 + b) * 16 + e) * 64] = acc[a][b][e];
        return;
    }
    // single slice: round to fp16 and store straight from the accumulators
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int gcol = col0 + nq * 64 + b * 32 + l32;
        if (gcol >= N)
            continue;
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int grow = row0 + a * 32 + (e >> 2) * 8 + h * 4 + (e & 3);
                if (grow < M)
                    d.C[(long)grow * N + gcol] = __builtin_bit_cast(uint16_t, (_Float16)acc[a][b][e]);
            }
    }
}

// Sums the split_k partial tiles of the skinny kernel in slice order and
// writes fp16 C.  Thread -> 4 consecutive floats of one tile's partial, which
// in the MFMA register layout are 4 adjacent columns of one output row.
__global__ __launch_bounds__(256) void reduce_partials_kernel(GroupTable tab, const float *partials)
{
    using namespace skinny;
    const long e = ((long)blockIdx.x * 256 + threadIdx.x) * 4;
    const int tile = (int)(e / kTileElems);
    const int idx = (int)(e - (long)tile * kTileElems);
    if (tile >= tab.prefix[tab.num_groups])
        return;
    const int S = tab.split_k;
    const int gi = find_group(tab, tile);
    const GemmDesc &d = tab.g[gi];
    const int r = tile - tab.prefix[gi];
    const int tm = r % d.tiles_m, tn = r / d.tiles_m;

    const float *src = partials + (long)tile * S * kTileElems + idx;
    float4 acc = *(const float4 *)src;
    for (int s = 1; s < S; ++s) {
        const float4 v = *(const float4 *)(src + (long)s * kTileElems);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    // register layout [nq][rb][cb][reg][lane] of the skinny kernel's partials
    const int lane0 = idx & 63;
    const int reg = (idx >> 6) & 15;
    const int cb = (idx >> 10) & 1;
    const int rb = (idx >> 11) & 1;
    const int nq = idx >> 12;
    const int row = tm * BM + rb * 32 + (reg >> 2) * 8 + (lane0 >> 5) * 4 + (reg & 3);
    const int col = tn * BN + nq * 64 + cb * 32 + (lane0 & 31);
    if (row >= d.M)
        return;
    uint16_t *dst = d.C + (long)row * d.N + col;
    const uint16_t v0 = __builtin_bit_cast(uint16_t, (_Float16)acc.x);
    const uint16_t v1 = __builtin_bit_cast(uint16_t, (_Float16)acc.y);
    const uint16_t v2 = __builtin_bit_cast(uint16_t, (_Float16)acc.z);
    const uint16_t v3 = __builtin_bit_cast(uint16_t, (_Float16)acc.w);
    if (col + 4 <= d.N && (((uintptr_t)dst) & 7) == 0) {
        *(u32x2 *)dst = (u32x2){(uint32_t)v0 | ((uint32_t)v1 << 16), (uint32_t)v2 | ((uint32_t)v3 << 16)};
    } else {
        if (col < d.N)
            dst[0] = v0;
        if (col + 1 < d.N)
            dst[1] = v1;
        if (col + 2 < d.N)
            dst[2] = v2;
        if (col + 3 < d.N)
            dst[3] = v3;
    }
}

} // namespace

hipError_t launch_grouped(const GroupTable &table, TileConfig cfg, void *workspace,
                          hipStream_t stream)
{
    const int tiles = table.prefix[table.num_groups];
    const int total = tiles * table.split_k;
    if (total <= 0)
        return hipSuccess;
    switch (cfg) {
    case kSkinny64x256: {
        float *partials = (float *)workspace;
        void *args[] = {const_cast<GroupTable *>(&table), &partials};
        bool vec = true;
        for (int g = 0; g < table.num_groups; ++g)
            vec = vec && (table.g[g].K % skinny::BK) == 0 && (((uintptr_t)table.g[g].SFB) & 15) == 0;
        const void *fn = vec ? (const void *)gemm_skinny_kernel<true> : (const void *)gemm_skinny_kernel<false>;
        hipError_t e = hipLaunchKernel(fn, dim3(total), dim3(skinny::kThreads), args, 0, stream);
        if (e != hipSuccess || table.split_k == 1)
            return e;
        const long threads = (long)tiles * skinny::kTileElems / 4;
        const float *cpart = partials;
        void *rargs[] = {const_cast<GroupTable *>(&table), &cpart};
        return hipLaunchKernel((const void *)reduce_partials_kernel, dim3((unsigned)((threads + 255) / 256)),
                               dim3(256), rargs, 0, stream);
    }
    case kTile128x128:
    default: {
        void *args[] = {const_cast<GroupTable *>(&table)};
        return hipLaunchKernel((const void *)gemm_tiled_kernel<128, 128, 128>, dim3(total),
                               dim3(256), args, 0, stream);
    }
    }
}

} // namespace nvfp4
