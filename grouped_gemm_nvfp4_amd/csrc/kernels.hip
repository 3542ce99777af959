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
    const int wave = tid >> 6;
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
        const __amdgpu_buffer_rsrc_t rs = (tid < 128) ? rSA : rSB;
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

} // namespace

hipError_t launch_grouped(const GroupTable &table, TileConfig cfg, void *workspace,
                          hipStream_t stream)
{
    (void)workspace;
    const int total = table.prefix[table.num_groups] * table.split_k;
    if (total <= 0)
        return hipSuccess;
    void *args[] = {const_cast<GroupTable *>(&table)};
    switch (cfg) {
    case kTile128x128:
    default:
        return hipLaunchKernel((const void *)gemm_tiled_kernel<128, 128, 128>, dim3(total),
                               dim3(256), args, 0, stream);
    }
}

} // namespace nvfp4
