// kernels.hip -- gfx950 (CDNA4) NVFP4 GEMM kernels staged through registers:
// the one- and four-wave 128 x 128 tiles for K % 128 != 0 or byte-path
// scales, the small-M stream and panel kernels with their in-kernel K-split
// sum, and the scale-layout conversion; the grouped launcher.  The
// direct-to-LDS 128 x 128 kernels are in kernels_dma.hip; the scale mapping
// and MFMA operand placement all kernels share are described in
// kernel_common.h.
#include "kernel_common.h"

namespace nvfp4 {
namespace {

// ---------------------------------------------------------------------------
// Tiled kernel: one workgroup of a single wave per 128 x 128 output tile.
// Four such workgroups share a CU (one per SIMD); each keeps its own LDS
// region, so no barrier is ever needed.
//
// Decode cost sets the tile: every 32x32x16 MFMA (32 cycles) needs an A and a
// B fragment of 8 elements per lane, 8 VALU instructions each (4 cvt + 4 mul,
// 4 cycles apiece on a 16-lane SIMD).  A wave owning a 128 x 128 tile decodes
// 4 A and 4 B fragments per 16 K and reuses them across 16 MFMAs: 4 VALU
// instructions per MFMA, half the MFMA time, issued in its shadow.
//
// Per K tile (128 elements): 20 loads per lane (A and B: 128 rows x 64 bytes;
// their 8 scale bytes per row) into registers one K tile ahead, then into the
// LDS stage; per 64-K group the lane reads 16 packed bytes of each of its 4 A
// rows and 4 B rows and runs 4 k-steps of 16 MFMAs.  LDS rows are 64 bytes
// with the 16-byte chunk index XORed with (row / 4) % 4, which makes both the
// row-wise writes and the MFMA-layout reads bank-conflict free, and keeps two
// stages at 36 KiB so that four workgroups fit a CU's 160 KiB.
// ---------------------------------------------------------------------------
struct TiledSlot {
    u32x4 a[8];   // A chunk c = 64 j + lane: row c / 4, bytes 16 (c % 4)
    u32x4 b[8];
    u32x2 sa[2];  // A scale rows lane and 64 + lane
    u32x2 sb[2];
};

// kVec: K % 128 == 0 and both scale arrays 8-byte aligned (one 8-byte load
// per row and K tile); otherwise 2-byte loads, pairs past K read as zero.
// kWaves (1 or 4): waves per workgroup.  With 4, the waves split the tile's K
// tiles four ways (one per SIMD of the CU, each with its own LDS stages) and
// their sums are added through LDS at the end: used when tiles alone would
// leave SIMDs idle.
// kWaves = 1: one wave owns a 128 x 128 tile.  kWaves = 4: four waves split
// each tile's K and add their sums through LDS.
template <bool kVec, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void gemm_tiled_kernel(GroupTable tab, float *partials, int *counters)
{
    using namespace tiled;
    __shared__ __attribute__((aligned(16))) uint8_t lds_all[kWaves * 2 * kStageBytes];

    const int wave = kWaves == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    uint8_t *lds = lds_all + wave * 2 * kStageBytes; // this wave's stages

    f32x16 acc[4][4];

    const int lane = (int)threadIdx.x & 63;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int crow = lane >> 2, c16 = lane & 3;
    const uint32_t sh = h * 16;

    // the tile and this wave's share [kb0, kb1) of its kt_tile K tiles
    const int w = blockIdx.x;
    const int gi = find_group(tab, w);
    const int kt_tile = (tab.g[gi].K + BK - 1) / BK;
    const int kb0 = (int)((long)kt_tile * wave / kWaves);
    const int kb1 = (int)((long)kt_tile * (wave + 1) / kWaves);
    const GemmDesc &d = tab.g[gi];
    const int r = w - tab.prefix[gi];
    const int tm = r % d.tiles_m;
    const int tn = r / d.tiles_m;
    const int M = d.M, N = d.N, K = d.K;
    const int row0 = tm * BM, col0 = tn * BN;

    const int kb_row = K / 2;
    const int ks_row = K / 16;
    const int kt_base = kb0;
    const int nkt = kb1 - kb0;
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(d.A + (long)row0 * kb_row, (uint64_t)(M - row0) * kb_row);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(d.B + (long)col0 * kb_row, (uint64_t)(N - col0) * kb_row);
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(d.SFA + (long)row0 * ks_row, (uint64_t)(M - row0) * ks_row);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(d.SFB + (long)col0 * ks_row, (uint64_t)(N - col0) * ks_row);
    const uint32_t line_off = (uint32_t)(crow * kb_row + c16 * 16);

    auto load = [&](TiledSlot &s, int kt) {
        const bool live = kt < nkt;
        const int kb = (kt_base + kt) * kRowBytes, ks = (kt_base + kt) * kSfBytes;
        const bool cin = live && (kb + c16 * 16) < kb_row; // chunk inside K
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t off = cin ? line_off + (uint32_t)(16 * j * kb_row + kb) : kOutOfRange;
            s.a[j] = __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0);
            s.b[j] = __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint32_t row = (uint32_t)(64 * j + lane);
            if (kVec) {
                const uint32_t off = live ? row * ks_row + ks : kOutOfRange;
                s.sa[j] = __builtin_amdgcn_raw_buffer_load_b64(rSA, off, 0, 0);
                s.sb[j] = __builtin_amdgcn_raw_buffer_load_b64(rSB, off, 0, 0);
            } else {
                uint32_t va[4], vb[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const bool ok = live && (ks + 2 * p) < ks_row;
                    const uint32_t off = ok ? row * ks_row + ks + 2 * p : kOutOfRange;
                    va[p] = __builtin_amdgcn_raw_buffer_load_b16(rSA, off, 0, 0);
                    vb[p] = __builtin_amdgcn_raw_buffer_load_b16(rSB, off, 0, 0);
                }
                s.sa[j] = (u32x2){va[0] | (va[1] << 16), va[2] | (va[3] << 16)};
                s.sb[j] = (u32x2){vb[0] | (vb[1] << 16), vb[2] | (vb[3] << 16)};
            }
        }
    };

    auto put = [&](const TiledSlot &s, int buf) {
        uint8_t *st = lds + buf * kStageBytes;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            *(u32x4 *)(st + kAOff + swz(16 * j + crow, c16)) = s.a[j];
            *(u32x4 *)(st + kBOff + swz(16 * j + crow, c16)) = s.b[j];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            *(u32x2 *)(st + kSaOff + (64 * j + lane) * kSfBytes) = s.sa[j];
            *(u32x2 *)(st + kSbOff + (64 * j + lane) * kSfBytes) = s.sb[j];
        }
    };

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = (f32x16){};

    // MFMA work of one 64-K group g of the tile in stage buf
    auto compute = [&](int buf, int g) {
        const uint8_t *st = lds + buf * kStageBytes;
        // scale pairs of this lane's half of group g: blocks 4g+2h, 4g+2h+1
        half2_t ca[4], cb[4];
        u32x4 pa[4], pb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x2 va = *(const u32x2 *)(st + kSaOff + (32 * i + l32) * kSfBytes);
            const u32x2 vb = *(const u32x2 *)(st + kSbOff + (32 * i + l32) * kSfBytes);
            ca[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((g ? va.y : va.x) >> sh, 1.0f, false);
            cb[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((g ? vb.y : vb.x) >> sh, 1.0f, false);
            pa[i] = *(const u32x4 *)(st + kAOff + swz(32 * i + l32, 2 * g + h));
            pb[i] = *(const u32x4 *)(st + kBOff + swz(32 * i + l32, 2 * g + h));
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            half8_t fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                fa[i] = decode8(pa[i][q], q < 2 ? bcast_lo(ca[i]) : bcast_hi(ca[i]));
                fb[i] = decode8(pb[i][q], q < 2 ? bcast_lo(cb[i]) : bcast_hi(cb[i]));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    };

    if (nkt > 0) {
        TiledSlot x;
        load(x, 0);
        put(x, 0);
        load(x, 1);
        for (int kt = 0; kt < nkt; ++kt) {
            // stage kt&1 holds tile kt; x holds tile kt + 1 (in flight).  The
            // refill sits between the two halves so that it issues while the
            // first half's MFMAs run.
            compute(kt & 1, 0);
            put(x, (kt + 1) & 1);
            load(x, kt + 2);
            compute(kt & 1, 1);
        }
    }

    if (kWaves > 1) {
        // add the waves' sums: 3 -> 1 and 2 -> 0, then 1 -> 0, through LDS in
        // register order ([reg][lane]: full 256-byte rows, conflict free)
        float *red = (float *)lds_all;
        constexpr int kAccFloats = 4 * 4 * 16 * 64;
        __syncthreads();
#pragma unroll
        for (int round = 0; round < 2; ++round) {
            const int give_lo = round == 0 ? 2 : 1; // waves [give_lo, 2 give_lo) hand over
            if (wave >= give_lo && wave < 2 * give_lo) {
                float *dst = red + (wave - give_lo) * kAccFloats + lane;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            dst[((i * 4 + j) * 16 + e) * 64] = acc[i][j][e];
            }
            __syncthreads();
            if (wave < give_lo) {
                const float *src = red + wave * kAccFloats + lane;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int e = 0; e < 16; ++e)
                            acc[i][j][e] += src[((i * 4 + j) * 16 + e) * 64];
            }
            __syncthreads();
        }
    }

    // epilogue: fp32 -> fp16 (round to nearest even) into LDS by wave 0, then
    // 16-byte row-contiguous stores masked to M x N by all waves.
    uint8_t *sC = lds_all;
    if (wave == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = 32 * i + (e >> 2) * 8 + h * 4 + (e & 3);
                    const int col = 32 * j + l32;
                    *(uint16_t *)(sC + row * kCStride + col * 2) =
                        __builtin_bit_cast(uint16_t, (_Float16)acc[i][j][e]);
                }
    }
    if (kWaves > 1)
        __syncthreads();
    const bool vec_ok = (N % 8 == 0) && ((((uintptr_t)d.C) & 15) == 0);
#pragma unroll 4
    for (int s = 0; s < BM * BN / 8 / (64 * kWaves); ++s) {
        const int seg = s * 64 * kWaves + (int)threadIdx.x;
        const int row = seg >> 4, c8 = (seg & 15) * 8;
        const int grow = row0 + row, gcol = col0 + c8;
        if (grow >= M)
            continue;
        uint16_t *dst = d.C + (long)grow * N + gcol;
        const uint16_t *src = (const uint16_t *)(sC + row * kCStride + c8 * 2);
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


// Last-arriver sum over the K slices of one output tile (split_k > 1).
// Every workgroup of the tile stores its partial values (kN per thread, at
// part + split * slice_elems + i * kStride) with agent-scope atomic stores,
// then takes a ticket from the tile's counter.  The workgroup that draws the
// last ticket adds the slices in slice order (so the result does not depend
// on arrival order), returns true with the sums in v, and resets the counter
// to zero for the next launch.  The others return false.  Every thread of the
// workgroup must call it.
//
// Ordering (HIP / HSA memory model): the barrier makes every thread's partial
// stores happen before thread 0's ticket, a fetch-add with release semantics
// at agent scope.  The fetch-adds on one counter form a release sequence, so
// the workgroup whose fetch-add returns S - 1 reads from every other
// workgroup's release; its acquire fence (agent scope) then makes all their
// partial stores visible to its loads after the second barrier.  The release
// costs one L2 write-back per workgroup and the acquire one L2 invalidate per
// output tile (last arriver only).
template <int kN, int kStride>
__device__ inline bool add_slices(float (&v)[kN], float *part, int slice_elems, int S, int split,
                                  int *counter, int *s_last)
{
#pragma unroll
    for (int i = 0; i < kN; ++i)
        __hip_atomic_store(part + (long)split * slice_elems + i * kStride, v[i], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (threadIdx.x == 0) {
        const bool last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == S - 1;
        if (last)
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        *s_last = last;
    }
    __syncthreads();
    if (!*s_last)
        return false;
    // slices in batches whose loads are all in flight before the first add
    constexpr int kBatch = 32 / kN;
    float t[kN];
    for (int s0 = 0; s0 < S; s0 += kBatch) {
        float x[kBatch][kN];
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            const int sl = s0 + b;
            if (sl < S && sl != split) {
#pragma unroll
                for (int i = 0; i < kN; ++i)
                    x[b][i] = __hip_atomic_load(part + (long)sl * slice_elems + i * kStride, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
            } else {
#pragma unroll
                for (int i = 0; i < kN; ++i)
                    x[b][i] = v[i];
            }
        }
#pragma unroll
        for (int b = 0; b < kBatch; ++b) {
            if (s0 + b < S) {
#pragma unroll
                for (int i = 0; i < kN; ++i)
                    t[i] = s0 + b == 0 ? x[b][i] : t[i] + x[b][i];
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kN; ++i)
        v[i] = t[i];
    if (threadIdx.x == 0)
        __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
}

// Two-slice sum without a ticket (split_k == 2 and pair slots given).  Each
// thread holds kN pairs of horizontally adjacent outputs, lo[i] and hi[i],
// and exchanges each pair (one 64-bit agent-scope atomic exchange) into its
// slot, slot + i * kStride pairs; between launches every slot holds
// kPairSentinel in both halves.  The exchange that gets a value back is the
// second one for that pair: it adds the two (fp32 addition of two terms is
// commutative, so the sum does not depend on which slice comes second and
// equals the slice-ordered sum), restores the sentinel for the next launch,
// and marks the pair as this thread's to write.  The pairing rests only on
// the atomicity of the two exchanges of one slot.
template <int kN, int kStride>
__device__ inline void add_pair(float (&lo)[kN], float (&hi)[kN], bool (&own)[kN], uint64_t *slot)
{
    constexpr uint64_t kEmpty = ((uint64_t)kPairSentinel << 32) | kPairSentinel;
    uint64_t old[kN];
#pragma unroll
    for (int i = 0; i < kN; ++i)
        old[i] = __hip_atomic_exchange(slot + i * kStride,
                                       ((uint64_t)__float_as_uint(hi[i]) << 32) | __float_as_uint(lo[i]),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
        own[i] = old[i] != kEmpty;
        if (own[i]) {
            lo[i] += __uint_as_float((uint32_t)old[i]);
            hi[i] += __uint_as_float((uint32_t)(old[i] >> 32));
            __hip_atomic_store(slot + i * kStride, kEmpty, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

namespace stream {
constexpr int BM = 64, BN = 32, BK = 256;
constexpr int kThreads = 512;
constexpr int kWaves = 8;
constexpr int kRowBytes = BK / 2;            // packed bytes per row per K tile
constexpr int kStride = kRowBytes + 16;      // padded LDS row
constexpr int kSfBytes = BK / 16;            // scale bytes per row per K tile
constexpr int kAOff = 0;
constexpr int kBOff = kAOff + BM * kStride;
constexpr int kSfaOff = kBOff + BN * kStride;
constexpr int kSfbOff = kSfaOff + BM * kSfBytes;
constexpr int kWaveBytes = kSfbOff + BN * kSfBytes; // 14848
constexpr int kTileElems = BM * BN;          // partial-sum floats per tile
static_assert(kWaves * kWaveBytes <= 160 * 1024, "wave regions must fit in LDS");
static_assert(kWaves * kTileElems * 4 <= kWaves * kWaveBytes, "reduction reuses the regions");
} // namespace stream

// One K tile of one wave, in registers: A 64 x 128 bytes as 8 lines of 8 rows,
// B 32 x 128 bytes as 4, and the scales of row lane (A) / lane % 32 (B).
struct StreamSlot {
    u32x4 a[8];
    u32x4 b[4];
    u32x4 sfa;
    u32x4 sfb;
};

// kVec: K % 256 == 0 and both scale arrays 16-byte aligned: a row's 16 scale
// bytes of a K tile are one aligned load.  Otherwise they are 8 two-byte
// loads (K % 32 == 0 makes each pair of blocks wholly inside or past K).
//
// kBlocked (with kVec): SFA and SFB in the blocked layout (512-byte atoms of
// 128 rows x 4 blocks, row r's block c of an atom at (r % 32) * 16 + (r / 32)
// * 4 + c).  A row's 16 scale bytes of a K tile are then one dword of each of
// the tile's four atoms: four 4-byte loads per operand, the tile's 64 A rows
// being one half of an atom's rows and its 32 B rows one quarter.
template <bool kVec, bool kBlocked>
__global__ __launch_bounds__(512) void gemm_stream_kernel(GroupTable tab, float *partials, int *counters)
{
    static_assert(kVec || !kBlocked, "blocked scales need K % 256 == 0");
    using namespace stream;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * kWaveBytes];
    __shared__ int s_last;

    const int S = tab.split_k;
    // XCD-contiguous runs of (tile, slice) pairs, as in the panel kernel
    // below.  Measured: 64 x 2048 x 2048 10.5 -> 9.8 us, 200 x 640 x 4096
    // 12.3 -> 11.6 us.
    int wg = (int)blockIdx.x;
    if ((gridDim.x & 7) == 0) {
        const int per = (int)(gridDim.x >> 3);
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int tile = wg / S;
    const int split = wg - tile * S;
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
    // this workgroup's K tiles, then this wave's share of them
    const int nkt = (K + BK - 1) / BK;
    const int s0 = (int)((long)split * nkt / S), s1 = (int)((long)(split + 1) * nkt / S);
    const int kt0 = s0 + (s1 - s0) * wave / kWaves;
    const int kt1 = s0 + (s1 - s0) * (wave + 1) / kWaves;

    // rows past M / N read as zero (beyond num_records)
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(d.A + (long)row0 * kb_row, (uint64_t)(M - row0) * kb_row);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(d.B + (long)col0 * kb_row, (uint64_t)(N - col0) * kb_row);
    // blocked: the 128-row atom band of the tile's rows (K / 64 atoms)
    const int rest_k = K / 64;
    const __amdgpu_buffer_rsrc_t rSA =
        kBlocked ? make_rsrc(d.SFA + (long)(row0 >> 7) * rest_k * 512, (uint64_t)rest_k * 512)
                 : make_rsrc(d.SFA + (long)row0 * ks_row, (uint64_t)(M - row0) * ks_row);
    const __amdgpu_buffer_rsrc_t rSB =
        kBlocked ? make_rsrc(d.SFB + (long)(col0 >> 7) * rest_k * 512, (uint64_t)rest_k * 512)
                 : make_rsrc(d.SFB + (long)col0 * ks_row, (uint64_t)(N - col0) * ks_row);

    // loop-invariant offsets: line loads cover rows 8j + lane/8, bytes 16 (lane%8)
    const int lrow = lane >> 3, c16 = lane & 7;
    const uint32_t line_off = (uint32_t)(lrow * kb_row + c16 * 16);
    // plain: row lane (A) / l32 (B) of the [rows][K/16] matrix; blocked: the
    // row's dword in an atom (A rows row0 % 128 + lane, B rows col0 % 128 + l32)
    const uint32_t sfa_off = kBlocked ? (uint32_t)((lane & 31) * 16 + (((row0 & 127) >> 5) + (lane >> 5)) * 4)
                                      : (uint32_t)(lane * ks_row);
    const uint32_t sfb_off = kBlocked ? (uint32_t)(l32 * 16 + ((col0 & 127) >> 5) * 4) : (uint32_t)(l32 * ks_row);

    auto load = [&](StreamSlot &s, int kt) {
        const bool live = kt < kt1;
        const int kb = kt * kRowBytes, ks = kt * kSfBytes;
        const bool cin = live && (kb + c16 * 16) < kb_row; // chunk inside K
#pragma unroll
        for (int j = 0; j < 8; ++j)
            s.a[j] = __builtin_amdgcn_raw_buffer_load_b128(
                rA, cin ? line_off + (uint32_t)(8 * j * kb_row + kb) : kOutOfRange, 0, 0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            s.b[j] = __builtin_amdgcn_raw_buffer_load_b128(
                rB, cin ? line_off + (uint32_t)(8 * j * kb_row + kb) : kOutOfRange, 0, 0);
        if (kBlocked) {
            // dword j of the row's 16 bytes: atom 4 kt + j
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t at = (uint32_t)((4 * kt + j) * 512);
                s.sfa[j] = __builtin_amdgcn_raw_buffer_load_b32(rSA, live ? at + sfa_off : kOutOfRange, 0, 0);
                s.sfb[j] = __builtin_amdgcn_raw_buffer_load_b32(rSB, live ? at + sfb_off : kOutOfRange, 0, 0);
            }
        } else if (kVec) {
            s.sfa = __builtin_amdgcn_raw_buffer_load_b128(rSA, live ? sfa_off + ks : kOutOfRange, 0, 0);
            s.sfb = __builtin_amdgcn_raw_buffer_load_b128(rSB, live ? sfb_off + ks : kOutOfRange, 0, 0);
        } else {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const bool ok0 = live && (ks + 4 * p) < ks_row;
                const bool ok1 = live && (ks + 4 * p + 2) < ks_row;
                const uint32_t a0 = __builtin_amdgcn_raw_buffer_load_b16(rSA, ok0 ? sfa_off + ks + 4 * p : kOutOfRange, 0, 0);
                const uint32_t a1 = __builtin_amdgcn_raw_buffer_load_b16(rSA, ok1 ? sfa_off + ks + 4 * p + 2 : kOutOfRange, 0, 0);
                const uint32_t b0 = __builtin_amdgcn_raw_buffer_load_b16(rSB, ok0 ? sfb_off + ks + 4 * p : kOutOfRange, 0, 0);
                const uint32_t b1 = __builtin_amdgcn_raw_buffer_load_b16(rSB, ok1 ? sfb_off + ks + 4 * p + 2 : kOutOfRange, 0, 0);
                s.sfa[p] = a0 | (a1 << 16);
                s.sfb[p] = b0 | (b1 << 16);
            }
        }
    };

    uint8_t *wl = lds + wave * kWaveBytes; // this wave's region

    auto put = [&](const StreamSlot &s) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *(u32x4 *)(wl + kAOff + (8 * j + lrow) * kStride + c16 * 16) = s.a[j];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *(u32x4 *)(wl + kBOff + (8 * j + lrow) * kStride + c16 * 16) = s.b[j];
        *(u32x4 *)(wl + kSfaOff + lane * kSfBytes) = s.sfa;
        if (h == 0)
            *(u32x4 *)(wl + kSfbOff + l32 * kSfBytes) = s.sfb;
    };

    f32x16 acc0 = (f32x16){}, acc1 = (f32x16){};
    const uint32_t sh = h * 16;

    auto compute = [&]() {
        const uint8_t *a0 = wl + kAOff + l32 * kStride + h * 16;
        const uint8_t *a1 = a0 + 32 * kStride;
        const uint8_t *b0 = wl + kBOff + l32 * kStride + h * 16;
        const u32x4 sa0 = *(const u32x4 *)(wl + kSfaOff + l32 * kSfBytes);
        const u32x4 sa1 = *(const u32x4 *)(wl + kSfaOff + (32 + l32) * kSfBytes);
        const u32x4 sb = *(const u32x4 *)(wl + kSfbOff + l32 * kSfBytes);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // this lane's half of 64-K group i: chunk 2i + h, blocks 4i+2h, 4i+2h+1
            const u32x4 pa0 = *(const u32x4 *)(a0 + i * 32);
            const u32x4 pa1 = *(const u32x4 *)(a1 + i * 32);
            const u32x4 pb = *(const u32x4 *)(b0 + i * 32);
            const half2_t ca0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa0[i] >> sh, 1.0f, false);
            const half2_t ca1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa1[i] >> sh, 1.0f, false);
            const half2_t cb = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb[i] >> sh, 1.0f, false);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const half8_t fa0 = decode8(pa0[q], q < 2 ? bcast_lo(ca0) : bcast_hi(ca0));
                const half8_t fa1 = decode8(pa1[q], q < 2 ? bcast_lo(ca1) : bcast_hi(ca1));
                const half8_t fb = decode8(pb[q], q < 2 ? bcast_lo(cb) : bcast_hi(cb));
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa0, fb, acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa1, fb, acc1, 0, 0, 0);
            }
        }
    };

    // step: move slot X (tile t) into LDS, refill it with tile t + 2, compute
    auto step = [&](int t, StreamSlot &X) {
        put(X);
        SCHED_FENCE();
        load(X, t + 2);
        SCHED_FENCE();
        if (t < kt1)
            compute();
        SCHED_FENCE();
    };

    if (kt1 > kt0) {
        StreamSlot x0, x1;
        load(x0, kt0);
        SCHED_FENCE();
        load(x1, kt0 + 1);
        SCHED_FENCE();
        for (int t = kt0; t < kt1; t += 2) {
            step(t, x0);
            if (t + 1 < kt1)
                step(t + 1, x1);
        }
    }

    // add the eight waves' partial sums through LDS (row-major 64 x 32 each)
    __syncthreads();
    float *red = (float *)lds;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int rr = (e >> 2) * 8 + h * 4 + (e & 3);
        red[wave * kTileElems + rr * BN + l32] = acc0[e];
        red[wave * kTileElems + (32 + rr) * BN + l32] = acc1[e];
    }
    __syncthreads();
    const int e0 = tid * 4; // 4 consecutive columns of one row
    float4 sum = *(const float4 *)(red + e0);
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        const float4 v = *(const float4 *)(red + w * kTileElems + e0);
        sum.x += v.x;
        sum.y += v.y;
        sum.z += v.z;
        sum.w += v.w;
    }
    if (S > 1) {
        // row-major partial tiles, [tile][slice][64][32]
        float vv[4] = {sum.x, sum.y, sum.z, sum.w};
        if (!add_slices<4, 1>(vv, partials + (long)tile * S * kTileElems + e0, kTileElems, S, split,
                              counters + tile, &s_last))
            return;
        sum = (float4){vv[0], vv[1], vv[2], vv[3]};
    }
    const int row = row0 + e0 / BN, col = col0 + e0 % BN;
    if (row >= M)
        return;
    uint16_t *dst = d.C + (long)row * N + col;
    const uint16_t v0 = __builtin_bit_cast(uint16_t, (_Float16)sum.x);
    const uint16_t v1 = __builtin_bit_cast(uint16_t, (_Float16)sum.y);
    const uint16_t v2 = __builtin_bit_cast(uint16_t, (_Float16)sum.z);
    const uint16_t v3 = __builtin_bit_cast(uint16_t, (_Float16)sum.w);
    if (col + 4 <= N && (((uintptr_t)dst) & 7) == 0) {
        *(u32x2 *)dst = (u32x2){(uint32_t)v0 | ((uint32_t)v1 << 16), (uint32_t)v2 | ((uint32_t)v3 << 16)};
    } else {
        if (col < N)
            dst[0] = v0;
        if (col + 1 < N)
            dst[1] = v1;
        if (col + 2 < N)
            dst[2] = v2;
        if (col + 3 < N)
            dst[3] = v3;
    }
}

// ----------------------------------------------------------------------------
// Small-M panel kernel: 64 x 64 tile per wave, operands staged through LDS.
//
// A workgroup owns a 64 x 64 output tile and a slice of K; its 8 waves split
// that slice again, each accumulating the whole 64 x 64 tile (four 32 x 32
// MFMA blocks) over its own share, and the 8 partial tiles are added through
// LDS at the end.  Per 16-K step a wave decodes four fragments (32 VALU) for
// four MFMAs, so decode and matrix work are balanced.
//
// Global loads are coalesced: per 256-K tile, eight lanes read one row's
// whole 128-byte line, 8 rows per instruction.  Each wave writes them into a
// private LDS region (no workgroup barrier in the K loop) and reads them back
// in MFMA lane order.  LDS rows are 128 bytes with the 16-byte chunk index
// XORed with (row / 2) % 8, which keeps both the row writes and the MFMA-order
// reads (16 lanes on 16 rows, same chunk) free of bank conflicts.
//
// MFMA step (i, q), i = 0..3, q = 0..3: lane half h supplies dword q of chunk
// 2i + h of its row, K [64i + 32h + 8q, +8), scale block 4i + 2h + q/2.
namespace panel {
constexpr int BM = 64, BN = 64, BK = 256;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBytes = BK / 2;  // 128
constexpr int kSfBytes = BK / 16;  // 16
constexpr int kAOff = 0;
constexpr int kBOff = kAOff + BM * kRowBytes;
constexpr int kSfaOff = kBOff + BN * kRowBytes;
constexpr int kSfbOff = kSfaOff + BM * kSfBytes;
constexpr int kWaveBytes = kSfbOff + BN * kSfBytes; // 18432
constexpr int kTileElems = BM * BN;
constexpr int kColStride = BM + 4; // floats per column of a partial tile (padded)
constexpr int kWaveFloats = BN * kColStride;
static_assert(kWaves * kWaveBytes <= 160 * 1024, "wave regions fit in LDS");
static_assert(kWaveFloats * 4 <= kWaveBytes, "partial tiles reuse the wave regions");
static_assert(kThreads * 8 == kTileElems, "8 outputs per thread in the final sum");
__device__ inline int swz(int r, int c) { return r * kRowBytes + ((c ^ ((r >> 1) & 7)) << 4); }
} // namespace panel

// One 256-K tile of one wave in registers: rows 8j + lane/8 of A and of B,
// bytes 16 (lane % 8) of their lines.  Scales travel separately.
struct PanelSlot {
    u32x4 a[8];
    u32x4 b[8];
};

// kVec: K % 256 == 0 and both scale arrays 16-byte aligned.  Then a wave
// fetches the scales of four K tiles at once, 64 contiguous bytes of 16 rows
// per instruction (lane l: row 16 i + l / 4, tile l % 4), and each tile's
// 16 bytes per row move to LDS when the tile does.  Otherwise the scales of
// each K tile are single-byte loads (lane l: row l), each masked against the
// row's K / 16 blocks.
//
// kBlocked (with kVec): SFA and SFB in the blocked layout, 512-byte atoms of
// 128 rows x 4 scale blocks (64 K), row r's block c of an atom at byte
// (r % 32) * 16 + (r / 32) * 4 + c.  A 64-row tile is one half of an atom's
// rows, so its scales of one atom are the 8-byte pieces at (r % 32) * 16 +
// 8 * half, each holding rows r % 32 and r % 32 + 32 of the tile.  A wave
// fetches the 16 atoms of four K tiles with 8 dwordx2 loads per operand
// (lane l: atom 2 i + l / 32 of the four tiles, line l % 32) and writes each
// tile's pieces into the same [row][16 bytes] LDS scale rows as the plain
// layout, dword j of a row being the tile's atom j.
//
// kMB: 32-row MFMA blocks of A that hold rows.  With kMB == 1 (every group
// of the launch has M <= 32, so rows 32..63 of the tile are past M) a wave
// loads, stores and decodes only rows 0..31 of A and issues two MFMAs per
// step instead of four; the other accumulators stay zero.
//
// With split_k > 1 every workgroup of a tile stores its partial tile, then
// takes a ticket from the tile's counter; the last to arrive adds all
// partial tiles in slice order (so the result does not depend on arrival
// order), writes C and resets the counter to zero for the next launch.
// With split_k == 2 and pair slots the two slices meet in the slots instead
// (add_pair), with no ticket or fence.
//
// kTail: some wave's count of K tiles is not a multiple of four, so the
// trips of four tiles end early; the staging writes and loads of the steps
// past a wave's last tile are skipped.  Launches whose every wave runs whole
// trips take the form without these checks (its schedule is the faster one
// there).
template <bool kVec, int kMB, bool kBlocked, bool kTail>
__global__ __launch_bounds__(panel::kThreads) void gemm_panel_kernel(GroupTable tab, float *partials, int *counters)
{
    static_assert(kMB == 1 || kMB == 2, "one or two 32-row blocks");
    static_assert(kVec || !kBlocked, "blocked scales take the four-tile scale groups");
    using namespace panel;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kWaves * kWaveBytes];
    __shared__ int s_last;

    const int S = tab.split_k;
    // Workgroups go to the eight XCDs round robin; with a grid that is a
    // multiple of 8, XCD x takes the contiguous run [x, x + 1) * grid / 8 of
    // (tile, slice) pairs, so the slices of a tile and neighbouring column
    // tiles (which share the 16-byte lines of blocked scale atoms) meet in
    // one L2.  Measured on 64 x 7168 x 16384: 30.5 -> 30.1 us plain, 31.3 ->
    // 30.5 us blocked.
    int wg = (int)blockIdx.x;
    if ((gridDim.x & 7) == 0) {
        const int per = (int)(gridDim.x >> 3);
        wg = (wg & 7) * per + (wg >> 3);
    }
    const int tile = wg / S;
    const int split = wg - tile * S;
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
    const int s0 = (int)((long)split * nkt / S), s1 = (int)((long)(split + 1) * nkt / S);
    const int kt0 = s0 + (s1 - s0) * wave / kWaves;
    const int kt1 = s0 + (s1 - s0) * (wave + 1) / kWaves;

    // rows past M / N read as zero (beyond num_records)
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(d.A + (long)row0 * kb_row, (uint64_t)(M - row0) * kb_row);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(d.B + (long)col0 * kb_row, (uint64_t)(N - col0) * kb_row);
    // blocked: the 128-row atom band holding the tile's rows (K % 256 == 0,
    // so K / 64 atoms per band)
    const int rest_k = K / 64;
    const __amdgpu_buffer_rsrc_t rSA =
        kBlocked ? make_rsrc(d.SFA + (long)(row0 >> 7) * rest_k * 512, (uint64_t)rest_k * 512)
                 : make_rsrc(d.SFA + (long)row0 * ks_row, (uint64_t)(M - row0) * ks_row);
    const __amdgpu_buffer_rsrc_t rSB =
        kBlocked ? make_rsrc(d.SFB + (long)(col0 >> 7) * rest_k * 512, (uint64_t)rest_k * 512)
                 : make_rsrc(d.SFB + (long)col0 * ks_row, (uint64_t)(N - col0) * ks_row);

    const int lrow = lane >> 3, c16 = lane & 7;
    const uint32_t line_off = (uint32_t)(lrow * kb_row + c16 * 16);
    const int grow = lane >> 2, gtile = lane & 3; // scale-group lane roles
    const uint32_t group_off = (uint32_t)(grow * ks_row + gtile * kSfBytes);

    auto load = [&](PanelSlot &s, int kt) {
        const int kb = kt * kRowBytes;
        // a 16-byte chunk is wholly inside or past the row's K / 2 bytes
        const bool cin = kt < kt1 && (kb + c16 * 16) < kb_row;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint32_t off = cin ? line_off + (uint32_t)(8 * j * kb_row + kb) : kOutOfRange;
            if (j < 4 * kMB)
                s.a[j] = __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0);
            s.b[j] = __builtin_amdgcn_raw_buffer_load_b128(rB, off, 0, 0);
        }
    };
    // vector path: scales of K tiles kt .. kt + 3 (tiles past this wave's
    // range read as zero)
    u32x4 gsa[4], gsb[4];
    auto load_group = [&](int kt) {
        const bool live = kt + gtile < kt1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = live ? group_off + (uint32_t)(16 * i * ks_row + kt * kSfBytes) : kOutOfRange;
            if (i < 2 * kMB)
                gsa[i] = __builtin_amdgcn_raw_buffer_load_b128(rSA, off, 0, 0);
            gsb[i] = __builtin_amdgcn_raw_buffer_load_b128(rSB, off, 0, 0);
        }
    };
    // blocked path: atoms of K tiles kt .. kt + 3, 8 bytes per lane
    u32x2 bsa[8], bsb[8];
    const uint32_t piece_a = (uint32_t)(l32 * 16 + ((row0 >> 6) & 1) * 8);
    const uint32_t piece_b = (uint32_t)(l32 * 16 + ((col0 >> 6) & 1) * 8);
    auto load_atoms = [&](int kt) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const bool live = kt + (i >> 1) < kt1;
            const uint32_t at = (uint32_t)((4 * kt + 2 * i + h) * 512);
            bsa[i] = __builtin_amdgcn_raw_buffer_load_b64(rSA, live ? at + piece_a : kOutOfRange, 0, 0);
            bsb[i] = __builtin_amdgcn_raw_buffer_load_b64(rSB, live ? at + piece_b : kOutOfRange, 0, 0);
        }
    };
    // general path: scales of K tile kt, row lane
    u32x4 tsa, tsb;
    auto load_bytes = [&](int kt) {
        const int ks = kt * kSfBytes;
        const bool live = kt < kt1;
        uint32_t va[4] = {0, 0, 0, 0}, vb[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const bool ok = live && (ks + i) < ks_row;
            const uint32_t off = ok ? (uint32_t)(lane * ks_row + ks + i) : kOutOfRange;
            va[i >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rSA, off, 0, 0) << (8 * (i & 3));
            vb[i >> 2] |= (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rSB, off, 0, 0) << (8 * (i & 3));
        }
        tsa = (u32x4){va[0], va[1], va[2], va[3]};
        tsb = (u32x4){vb[0], vb[1], vb[2], vb[3]};
    };

    uint8_t *wl = lds + wave * kWaveBytes; // this wave's region

    // data of the tile in `s` and its scales (group slot u on the vector path)
    auto put = [&](const PanelSlot &s, int u) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < 4 * kMB)
                *(u32x4 *)(wl + kAOff + swz(8 * j + lrow, c16)) = s.a[j];
            *(u32x4 *)(wl + kBOff + swz(8 * j + lrow, c16)) = s.b[j];
        }
        if (kBlocked) {
            // tile u: loads 2u (atoms 0, 1 by lane half) and 2u + 1 (atoms 2, 3)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int j = 2 * e + h;
                const u32x2 pa = bsa[2 * u + e], pb = bsb[2 * u + e];
                *(uint32_t *)(wl + kSfaOff + l32 * kSfBytes + 4 * j) = pa[0];
                if (kMB == 2)
                    *(uint32_t *)(wl + kSfaOff + (32 + l32) * kSfBytes + 4 * j) = pa[1];
                *(uint32_t *)(wl + kSfbOff + l32 * kSfBytes + 4 * j) = pb[0];
                *(uint32_t *)(wl + kSfbOff + (32 + l32) * kSfBytes + 4 * j) = pb[1];
            }
        } else if (kVec) {
            if (gtile == u) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if (i < 2 * kMB)
                        *(u32x4 *)(wl + kSfaOff + (16 * i + grow) * kSfBytes) = gsa[i];
                    *(u32x4 *)(wl + kSfbOff + (16 * i + grow) * kSfBytes) = gsb[i];
                }
            }
        } else {
            *(u32x4 *)(wl + kSfaOff + lane * kSfBytes) = tsa;
            *(u32x4 *)(wl + kSfbOff + lane * kSfBytes) = tsb;
        }
    };

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = (f32x16){};
    const uint32_t sh = h * 16;

    auto compute = [&]() {
        u32x4 sa[2], sb[2]; // the 16 scale bytes of rows 32 o + l32
#pragma unroll
        for (int o = 0; o < 2; ++o) {
            if (o < kMB)
                sa[o] = *(const u32x4 *)(wl + kSfaOff + (32 * o + l32) * kSfBytes);
            sb[o] = *(const u32x4 *)(wl + kSfbOff + (32 * o + l32) * kSfBytes);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 pa[2], pb[2];
            half2_t ca[2], cb[2]; // blocks 4i + 2h (.x) and 4i + 2h + 1 (.y)
#pragma unroll
            for (int o = 0; o < 2; ++o) {
                if (o < kMB)
                    pa[o] = *(const u32x4 *)(wl + kAOff + swz(32 * o + l32, 2 * i + h));
                pb[o] = *(const u32x4 *)(wl + kBOff + swz(32 * o + l32, 2 * i + h));
                if (o < kMB)
                    ca[o] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa[o][i] >> sh, 1.0f, false);
                cb[o] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sb[o][i] >> sh, 1.0f, false);
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                half8_t fa[2], fb[2];
#pragma unroll
                for (int o = 0; o < 2; ++o) {
                    if (o < kMB)
                        fa[o] = decode8(pa[o][q], q < 2 ? bcast_lo(ca[o]) : bcast_hi(ca[o]));
                    fb[o] = decode8(pb[o][q], q < 2 ? bcast_lo(cb[o]) : bcast_hi(cb[o]));
                }
#pragma unroll
                for (int oa = 0; oa < kMB; ++oa)
#pragma unroll
                    for (int ob = 0; ob < 2; ++ob)
                        acc[oa][ob] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[oa], fb[ob], acc[oa][ob], 0, 0, 0);
            }
        }
    };

    if (kt1 > kt0) {
        PanelSlot x;
        load(x, kt0);
        if (kBlocked)
            load_atoms(kt0);
        else if (kVec)
            load_group(kt0);
        else
            load_bytes(kt0);
        SCHED_FENCE();
        // four K tiles per trip, one per scale-group slot; steps past kt1 skip
        // the compute (and with kTail the staging and the next load)
        for (int t = kt0; t < kt1; t += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if constexpr (kTail) {
                    if (t + u < kt1)
                        put(x, u);
                } else {
                    put(x, u);
                }
                SCHED_FENCE();
                if constexpr (kTail) {
                    if (t + u + 1 < kt1)
                        load(x, t + u + 1);
                } else {
                    load(x, t + u + 1);
                }
                if (kBlocked) {
                    if (u == 3)
                        load_atoms(t + 4);
                } else if (kVec) {
                    if (u == 3)
                        load_group(t + 4);
                } else {
                    load_bytes(t + u + 1);
                }
                SCHED_FENCE();
                if (t + u < kt1)
                    compute();
                SCHED_FENCE();
            }
        }
    }

    // every wave is done with its staging region before the partial tiles
    // (which overlap other waves' regions) are written
    __syncthreads();
    float *red = (float *)lds;
    // column-major with padded columns: lane l holds rows 32 oa + 8 g + 4 h
    // + (0..3) of column 32 ob + l % 32
    float *mine = red + wave * kWaveFloats;
#pragma unroll
    for (int oa = 0; oa < 2; ++oa)
#pragma unroll
        for (int ob = 0; ob < 2; ++ob)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                *(float4 *)(mine + (32 * ob + l32) * kColStride + 32 * oa + 8 * g + 4 * h) =
                    (float4){acc[oa][ob][4 * g], acc[oa][ob][4 * g + 1], acc[oa][ob][4 * g + 2], acc[oa][ob][4 * g + 3]};
    __syncthreads();

    // thread -> columns n, n + 1 (n = 2 (tid % 32)), rows 4 (tid / 32) .. + 3,
    // summed in wave order: lo[r], hi[r] are row m0 + r of columns n, n + 1
    const int n = (tid & 31) * 2, m0 = (tid >> 5) * 4;
    float lo[4], hi[4];
    {
        const float4 p = *(const float4 *)(red + n * kColStride + m0);
        const float4 q = *(const float4 *)(red + (n + 1) * kColStride + m0);
        lo[0] = p.x; lo[1] = p.y; lo[2] = p.z; lo[3] = p.w;
        hi[0] = q.x; hi[1] = q.y; hi[2] = q.z; hi[3] = q.w;
    }
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        const float4 p = *(const float4 *)(red + w * kWaveFloats + n * kColStride + m0);
        const float4 q = *(const float4 *)(red + w * kWaveFloats + (n + 1) * kColStride + m0);
        lo[0] += p.x; lo[1] += p.y; lo[2] += p.z; lo[3] += p.w;
        hi[0] += q.x; hi[1] += q.y; hi[2] += q.z; hi[3] += q.w;
    }
    bool own[4] = {true, true, true, true}; // the pairs this thread writes
    if (S == 2 && tab.pairs != nullptr) {
        // pair slots, row-major [tile][64][64] floats, one 64-bit slot per
        // two adjacent columns
        add_pair<4, BN / 2>(lo, hi, own, (uint64_t *)(tab.pairs + (long)tile * kTileElems + m0 * BN + n));
    } else if (S > 1) {
        // partial tiles [tile][slice][8][kThreads]: value i of thread t at
        // i * kThreads + t
        float v[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if (!add_slices<8, kThreads>(v, partials + (long)tile * S * kTileElems + tid, kTileElems, S, split,
                                     counters + tile, &s_last))
            return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            lo[r] = v[r];
            hi[r] = v[4 + r];
        }
    }
    const int col = col0 + n;
    if (col >= N)
        return;
    // two adjacent outputs as one 4-byte store where both lie inside N and
    // the address is 4-byte aligned
    const bool pair_store = col + 1 < N && (N & 1) == 0 && (((uintptr_t)d.C) & 3) == 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = row0 + m0 + r;
        if (!own[r] || row >= M)
            continue;
        uint16_t *dst = d.C + (long)row * N + col;
        const uint16_t a = __builtin_bit_cast(uint16_t, (_Float16)lo[r]);
        const uint16_t b = __builtin_bit_cast(uint16_t, (_Float16)hi[r]);
        if (pair_store) {
            *(uint32_t *)dst = (uint32_t)a | ((uint32_t)b << 16);
        } else {
            dst[0] = a;
            if (col + 1 < N)
                dst[1] = b;
        }
    }
}

// ----------------------------------------------------------------------------
// Scale layout conversion (see ScaleConvTable).  A workgroup of 256 threads
// takes one 128-row tile and kConvAtoms consecutive atoms (4 KiB): the blocked
// side moves as coalesced 16-byte lane pieces, the plain side through LDS as
// 16-byte row pieces (bytes, as plain rows start at any byte).
__global__ __launch_bounds__(256) void scale_conversion_kernel(ScaleConvTable tab)
{
    __shared__ __attribute__((aligned(16))) uint8_t atoms[kConvAtoms * 512];
    const int wgi = (int)blockIdx.x;
    int lo = 0, hi = tab.count;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tab.prefix[mid] <= wgi)
            lo = mid;
        else
            hi = mid;
    }
    const int e = lo;
    const int kb = tab.kb[e], rows = tab.rows[e];
    const int rest_k = (kb + 3) / 4;
    const int runs = (rest_k + kConvAtoms - 1) / kConvAtoms;
    const int local = wgi - tab.prefix[e];
    const int tm = local / runs, t0 = (local - tm * runs) * kConvAtoms;
    const int natoms = min(kConvAtoms, rest_k - t0);
    const int tid = threadIdx.x;
    // blocked side: thread -> atom tid / 32, 16-byte piece tid % 32
    const int pa = tid >> 5, pp = tid & 31;
    const long blk_off = ((long)tm * rest_k + t0 + pa) * 512 + pp * 16;
    // plain side: thread -> row tid / 2, blocks [16 (tid % 2), +16) of the run
    const int r = tid >> 1, jh = (tid & 1) * 16;
    const int m = tm * 128 + r;
    auto lds_byte = [&](int j) -> uint8_t & { // block j (0..31) of row r in the run
        return atoms[(j >> 2) * 512 + (r % 32) * 16 + (r / 32) * 4 + (j & 3)];
    };
    // the thread's 16 plain bytes as one 16-byte access when they are whole
    // and 16-byte aligned (K % 256 == 0 and an aligned base), else bytes
    const uint8_t *plain_in = tab.to_blocked ? tab.src[e] : nullptr;
    uint8_t *plain_out = tab.to_blocked ? nullptr : tab.dst[e];
    const long plain_off = (long)m * kb + 4 * t0 + jh;
    const bool whole = m < rows && 4 * t0 + jh + 16 <= kb &&
                       (((uintptr_t)(tab.to_blocked ? (const void *)plain_in : (const void *)plain_out) + plain_off) & 15) == 0;
    if (tab.to_blocked) {
        if (whole) {
            const u32x4 v = *(const u32x4 *)(plain_in + plain_off);
#pragma unroll
            for (int j = 0; j < 16; ++j)
                lds_byte(jh + j) = (uint8_t)(v[j >> 2] >> (8 * (j & 3)));
        } else {
            const uint8_t *src = plain_in + (long)m * kb;
#pragma unroll
            for (int j = jh; j < jh + 16; ++j) {
                const int blk = 4 * t0 + j;
                lds_byte(j) = (m < rows && blk < kb) ? src[blk] : 0;
            }
        }
        __syncthreads();
        if (pa < natoms)
            *(u32x4 *)(tab.dst[e] + blk_off) = *(const u32x4 *)(atoms + pa * 512 + pp * 16);
    } else {
        if (pa < natoms)
            *(u32x4 *)(atoms + pa * 512 + pp * 16) = *(const u32x4 *)(tab.src[e] + blk_off);
        __syncthreads();
        if (whole) {
            u32x4 v = (u32x4){0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 16; ++j)
                v[j >> 2] |= (uint32_t)lds_byte(jh + j) << (8 * (j & 3));
            *(u32x4 *)(plain_out + plain_off) = v;
        } else if (m < rows) {
            uint8_t *dst = plain_out + (long)m * kb;
#pragma unroll
            for (int j = jh; j < jh + 16; ++j) {
                const int blk = 4 * t0 + j;
                if (blk < kb)
                    dst[blk] = lds_byte(j);
            }
        }
    }
}

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *p, int words)
{
    for (int i = (int)threadIdx.x; i < words; i += 256)
        p[i] = 0;
}

} // namespace

hipError_t launch_clear_words(void *p, int words, hipStream_t stream)
{
    if (words <= 0)
        return hipSuccess;
    uint32_t *q = (uint32_t *)p;
    void *args[] = {&q, &words};
    return hipLaunchKernel((const void *)clear_words_kernel, dim3(1), dim3(256), args, 0, stream);
}

// True when some wave of a panel launch has a K-tile count that is not a
// multiple of four: a slice of L K tiles gives its eight waves L (w + 1) / 8
// - L w / 8 tiles each, all multiples of four exactly when L % 32 == 0.
bool panel_tail(const GroupTable &table)
{
    const int S = table.split_k;
    for (int g = 0; g < table.num_groups; ++g) {
        const int nkt = (table.g[g].K + panel::BK - 1) / panel::BK;
        if (nkt % S != 0 || (nkt / S) % (4 * panel::kWaves) != 0)
            return true;
    }
    return false;
}

hipError_t launch_grouped(const GroupTable &table, TileConfig cfg, int *counters, float *partials,
                          hipStream_t stream)
{
    const int tiles = table.prefix[table.num_groups];
    const int total = tiles * table.split_k;
    if (total <= 0)
        return hipSuccess;
    if (table.split_k > 1 && (counters == nullptr || partials == nullptr || tiles > kMaxSplitTiles))
        return hipErrorInvalidValue;
    // the pair slots hold one 64 x 64 tile's elements per tile
    if (table.pairs != nullptr && table.split_k == 2 && (long long)tiles * 64 * 64 * 4 > kPairSlotBytes)
        return hipErrorInvalidValue;
    void *args[] = {const_cast<GroupTable *>(&table), &partials, &counters};
    switch (cfg) {
    case kStream64x32: {
        bool vec = true;
        for (int g = 0; g < table.num_groups; ++g)
            vec = vec && (table.g[g].K % stream::BK) == 0 &&
                  ((((uintptr_t)table.g[g].SFA) | ((uintptr_t)table.g[g].SFB)) & 15) == 0;
        const void *fn = vec ? (const void *)gemm_stream_kernel<true, false> : (const void *)gemm_stream_kernel<false, false>;
        return hipLaunchKernel(fn, dim3(total), dim3(stream::kThreads), args, 0, stream);
    }
    case kPanel64x64: {
        bool vec = true;
        for (int g = 0; g < table.num_groups; ++g)
            vec = vec && (table.g[g].K % panel::BK) == 0 &&
                  ((((uintptr_t)table.g[g].SFA) | ((uintptr_t)table.g[g].SFB)) & 15) == 0;
        // rows 32..63 of every tile past M: the one-block form
        bool half = true;
        for (int g = 0; g < table.num_groups; ++g)
            half = half && table.g[g].M <= 32;
        const bool tail = panel_tail(table);
        const void *fn;
        if (tail)
            fn = half ? (vec ? (const void *)gemm_panel_kernel<true, 1, false, true>
                             : (const void *)gemm_panel_kernel<false, 1, false, true>)
                      : (vec ? (const void *)gemm_panel_kernel<true, 2, false, true>
                             : (const void *)gemm_panel_kernel<false, 2, false, true>);
        else
            fn = half ? (vec ? (const void *)gemm_panel_kernel<true, 1, false, false>
                             : (const void *)gemm_panel_kernel<false, 1, false, false>)
                      : (vec ? (const void *)gemm_panel_kernel<true, 2, false, false>
                             : (const void *)gemm_panel_kernel<false, 2, false, false>);
        return hipLaunchKernel(fn, dim3(total), dim3(panel::kThreads), args, 0, stream);
    }
    case kStream64x32Blocked: {
        // blocked scales: every K % 256 == 0 and SFA, SFB 16-byte aligned
        for (int g = 0; g < table.num_groups; ++g)
            if (table.g[g].K % stream::BK != 0 || (((uintptr_t)table.g[g].SFA) | ((uintptr_t)table.g[g].SFB)) & 15)
                return hipErrorInvalidValue;
        return hipLaunchKernel((const void *)gemm_stream_kernel<true, true>, dim3(total), dim3(stream::kThreads), args,
                               0, stream);
    }
    case kPanel64x64Blocked: {
        // blocked scales: every K % 256 == 0 and SFA, SFB 16-byte aligned
        bool half = true;
        for (int g = 0; g < table.num_groups; ++g) {
            if (table.g[g].K % panel::BK != 0 || (((uintptr_t)table.g[g].SFA) | ((uintptr_t)table.g[g].SFB)) & 15)
                return hipErrorInvalidValue;
            half = half && table.g[g].M <= 32;
        }
        const bool tail = panel_tail(table);
        const void *fn = tail ? (half ? (const void *)gemm_panel_kernel<true, 1, true, true>
                                      : (const void *)gemm_panel_kernel<true, 2, true, true>)
                              : (half ? (const void *)gemm_panel_kernel<true, 1, true, false>
                                      : (const void *)gemm_panel_kernel<true, 2, true, false>);
        return hipLaunchKernel(fn, dim3(total), dim3(panel::kThreads), args, 0, stream);
    }
    case kTile128x128K4:
    case kTile128x128Pow2:
    case kTile128x128Blocked:
    case kTile128x128:
    default: {
        bool vec = true;
        for (int g = 0; g < table.num_groups; ++g)
            vec = vec && (table.g[g].K % tiled::BK) == 0 &&
                  ((((uintptr_t)table.g[g].SFA) | ((uintptr_t)table.g[g].SFB)) & 7) == 0;
        if (cfg == kTile128x128Blocked || cfg == kTile128x128Pow2 || vec)
            return launch_tiled_dma(table, cfg, stream);
        // K % 128 != 0 or byte-path scales: the K tile goes through registers
        const bool four = cfg == kTile128x128K4;
        const void *fn = four ? (const void *)gemm_tiled_kernel<false, 4> : (const void *)gemm_tiled_kernel<false, 1>;
        return hipLaunchKernel(fn, dim3(tiles), dim3(four ? 256 : 64), args, 0, stream);
    }
    }
}

hipError_t launch_scale_conversion(const ScaleConvTable &table, hipStream_t stream)
{
    const int wgs = table.prefix[table.count];
    if (wgs <= 0)
        return hipSuccess;
    void *args[] = {const_cast<ScaleConvTable *>(&table)};
    return hipLaunchKernel((const void *)scale_conversion_kernel, dim3((unsigned)wgs), dim3(256), args, 0, stream);
}

} // namespace nvfp4
