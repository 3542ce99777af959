// kernel_common.h -- what the gfx950 (CDNA4) NVFP4 GEMM kernels share.
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
#pragma once

#include "launch.h"

namespace nvfp4 {
namespace {


typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)

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

// A problem table read from device memory (device-resident grouped calls).
struct DevTableView {
    int num_groups;
    const int *prefix;
    const GemmDesc *g;
};

// Workgroup -> (group, tile) through the exclusive prefix over tile counts
// (the last group whose prefix entry is <= w: empty groups are passed over).
template <class Table>
__device__ inline int find_group(const Table &t, int w)
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

namespace tiled {
constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kRowBytes = BK / 2;          // 64 packed bytes per row per K tile
constexpr int kStride = kRowBytes;         // swizzled, unpadded LDS row
constexpr int kSfBytes = BK / 16;          // 8 scale bytes per row per K tile
constexpr int kAOff = 0;
constexpr int kBOff = BM * kStride;
constexpr int kSaOff = kBOff + BN * kStride;
constexpr int kSbOff = kSaOff + BM * kSfBytes;
constexpr int kStageBytes = kSbOff + BN * kSfBytes; // 18432
// byte offset of 16-byte chunk c of row r within an A or B stage
__device__ inline int swz(int r, int c) { return r * kStride + ((c ^ ((r >> 2) & 3)) << 4); }
constexpr int kCStride = BN * 2 + 16;      // bytes per fp16 C row in LDS
static_assert(2 * kStageBytes >= BM * kCStride, "C tile reuses the stages");
} // namespace tiled

} // namespace
} // namespace nvfp4
