/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 block-scaled GEMM library.
 *
 * The operation (kernelbot pages nvfp4-group-gemm-498453 and nvfp4-gemm-125598,
 * `custom_kernel` docstrings and the block-scaled MMA loop: C = A * SFA * B * SFB
 * with sf_vec_size 16):
 *
 *     C[m][n] = fp16_rne( sum_{k<K} (A[m][k] * SFA[m][k/16]) * (B[n][k] * SFB[n][k/16]) )
 *
 * accumulated in fp32 (the pages' Float32 accumulator) and rounded to binary16
 * with round-to-nearest-even (the raw-CUDA page nvfp4-group-gemm-407526, epilogue,
 * `__floats2half2_rn`).  Overflow gives +-inf.
 *
 * Operand layouts (all dense, row-major, device memory, caller-owned):
 *   A   [M][K/2]   uint8: two FP4 E2M1 codes per byte along K, the LOW nibble
 *                  holds the even k (torch float4_e2m1fn_x2 of shape [M, K/2]).
 *   SFA [M][K/16]  uint8: FP8 E4M3 ("fn": bias 7, max 448, no inf) scale codes,
 *                  one per 16 consecutive K elements of a row.
 *   B   [N][K/2]   uint8, SFB [N][K/16] uint8: the same for the second operand
 *                  (B is stored N-major, K contiguous, as on the pages).
 *   C   [M][N]     IEEE binary16, written in full by the call.
 * A and B must be 16-byte aligned (the kernels move them in 16-byte loads);
 * SFA, SFB and C need only their natural alignment.  C must not alias any
 * input.
 *
 * Calls are asynchronous on `stream` (NULL = the device's null stream): C is
 * valid once the stream has reached the call.  The calling thread's current
 * HIP device must own every buffer.  Nothing is printed; no exception crosses
 * the boundary.  Argument errors are reported before any HIP call is made.
 *
 * Threads: the calls may be made from several threads.  Calls that split K
 * use a device workspace that the library keeps per (device, stream) pair
 * (per calling thread as well for hipStreamPerThread) and grows on demand
 * (hipMalloc plus one initialisation of its tile counters and two-slice
 * pair slots, enqueued on the stream before the call's kernels; every call
 * leaves them as it found them); calls on one stream are ordered by that
 * stream, so they never share a workspace concurrently.
 *
 * Stream capture: a call that would have to allocate or grow its stream's
 * workspace while that stream is capturing returns NVFP4_ERROR_NOT_SUPPORTED
 * and enqueues nothing; one eager call of the same or a larger size on the
 * stream beforehand makes the captured call possible.  A captured K-split
 * call keeps using the workspace of the stream it was captured on: its graph
 * must not run at the same time as other work that uses that workspace (eager
 * calls on that stream, or other replays of graphs captured on it).
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 1
/* Largest number of groups a single grouped call accepts. */
#define NVFP4_MAX_GROUPS 4096
/* Largest K of a product.  The kernels accumulate in fp32; an output's
 * longest serial chain is K / 16 matrix-core steps plus at most a few dozen
 * sums of partial results.  Counting two roundings per step, each at most
 * 2^-24 of a partial sum no larger than sum_k |a_k b_k|, the accumulated error
 * stays below K * 2^-27 * sum_k |a_k b_k| + 2^-19 * sum_k |a_k b_k|, which is
 * inside the 1e-3 * sum_k |a_k b_k| accuracy bound for every K up to this. */
#define NVFP4_MAX_K 131072

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERROR_INVALID_VALUE = 1, /* null pointer, negative size, bad group count */
    NVFP4_ERROR_NOT_SUPPORTED = 2, /* K not a multiple of 32, sizes beyond int32 tiling */
    NVFP4_ERROR_LAUNCH = 3,        /* a HIP call failed (launch, workspace allocation) */
} nvfp4_status;

/* One independent product of a grouped call. */
typedef struct {
    const void *A;   /* [M][K/2] packed e2m1 */
    const void *SFA; /* [M][K/16] e4m3 */
    const void *B;   /* [N][K/2] packed e2m1 */
    const void *SFB; /* [N][K/16] e4m3 */
    void *C;         /* [M][N] binary16 */
    int M, N, K;
} nvfp4_problem;

/*
 * Single NVFP4 GEMM (the single-GEMM page nvfp4-gemm-125598, `custom_kernel`,
 * with its batch size l fixed at 1).
 *   M, N >= 0; K >= 0 and K % 32 == 0.  M == 0 or N == 0: nothing is done.
 *   K == 0: C is filled with +0 (the empty sum).
 * Errors: any pointer NULL while M*N > 0 (A/SFA/B/SFB only when K > 0)
 *   -> NVFP4_ERROR_INVALID_VALUE; negative sizes -> INVALID_VALUE;
 *   K % 32 != 0, K > NVFP4_MAX_K, A or B not 16-byte aligned, or more than
 *   2^24 - 1 workgroups -> NVFP4_ERROR_NOT_SUPPORTED;
 *   a failed launch or workspace allocation -> NVFP4_ERROR_LAUNCH.
 */
nvfp4_status nvfp4_gemm(const void *A, const void *SFA, const void *B, const void *SFB,
                        void *C, int M, int N, int K, hipStream_t stream);

/*
 * Grouped NVFP4 GEMM: num_groups independent products in one launch (the
 * grouped pages nvfp4-group-gemm-407526 `group_gemm` and
 * nvfp4-group-gemm-498453 `custom_kernel`: per-group A, B, C, SFA, SFB and
 * (m, n, k, l) with l = 1).  Work is scheduled by an exclusive prefix sum over
 * the groups' output-tile counts; a workgroup finds its group by searching that
 * prefix (the CuTeDSL grouped page, group lookup from the CTA index).
 *   `problems` is a host array of num_groups entries, read during the call only.
 *   Up to 64 non-empty groups go into one launch; more are issued as several
 *   launches on the same stream.
 *   0 <= num_groups <= NVFP4_MAX_GROUPS; num_groups == 0 is a no-op.
 *   Each group obeys the single-GEMM rules above (empty groups are skipped).
 * Errors: as nvfp4_gemm, per group; problems == NULL with num_groups > 0 or
 *   num_groups outside [0, NVFP4_MAX_GROUPS] -> NVFP4_ERROR_INVALID_VALUE.
 *   On an argument error nothing is launched for any group.
 */
nvfp4_status nvfp4_group_gemm(const nvfp4_problem *problems, int num_groups,
                              hipStream_t stream);

/* ---- Batch l > 1 (the pages' (m, n, k, l) problems: the grouped page
 * nvfp4-group-gemm-498453, `custom_kernel` docstring and problem sizes; the
 * single-GEMM page nvfp4-gemm-125598, `custom_kernel` and the tensor layouts
 * (m, k, l) with strides (k, 1, m k)): L products of the same sizes whose
 * operands are dense stacks, batch b of A at A + b M K/2 bytes, SFA + b M K/16,
 * B + b N K/2, SFB + b N K/16, C + b M N elements.  Runs as one grouped call.
 *   0 <= L <= NVFP4_MAX_GROUPS (more: NOT_SUPPORTED; negative: INVALID_VALUE);
 *   L == 0 is a no-op.  Each batch obeys the single-GEMM rules above. */
nvfp4_status nvfp4_gemm_batched(const void *A, const void *SFA, const void *B, const void *SFB,
                                void *C, int M, int N, int K, int L, hipStream_t stream);

/* ---- Device-resident problem tables (the grouped page nvfp4-group-gemm-498453
 * keeps the per-group sizes, pointers and the CTA prefix in device tensors,
 * `custom_kernel` host code and the group lookup in the kernel).  For callers
 * whose group sizes are produced on the device (an MoE router's per-expert row
 * counts) or who replay the call in a captured graph with sizes that change
 * between replays.
 *
 * `problems` is a DEVICE array of num_groups nvfp4_problem entries, read by
 * the enqueued work (not by this call), so it may be written by earlier work
 * on the stream.  A one-workgroup plan kernel checks every entry, computes
 * the per-group 128 x 128 tile counts and their prefix into `workspace`, then
 * a grid of max_tiles one-wave workgroups runs the tiles (workgroups past the
 * table's total return at once).  No allocation, no host synchronisation, no
 * memset: the call can be captured in a HIP graph.
 *
 * Per-entry contract, checked on the device: M, N, K >= 0; K % 128 == 0 and
 * K <= NVFP4_MAX_K; when M N > 0, C present and, when K > 0, A, SFA, B, SFB present
 * with A and B 16-byte and SFA and SFB 8-byte aligned; at most 2^24 tiles.
 * An entry outside it gets no tiles (its C is not written) and is counted.
 * After the work has run, the workspace starts with four int32: num_groups,
 * the tiles the table asked for (clamped to INT32_MAX), the number of entries
 * outside the contract, 0.  Tiles past max_tiles (total > max_tiles) are not
 * computed: the caller bounds max_tiles from above (for an MoE layer,
 * (tokens * top_k / 128 + num_groups) * ceil(N / 128)).
 *
 * workspace: device memory of at least
 * nvfp4_group_gemm_device_workspace_bytes(num_groups) bytes, 16-byte aligned,
 * owned by the caller; calls that overlap in time must not share it.
 * Errors (host, before any HIP call): num_groups outside [0,
 * NVFP4_MAX_GROUPS], max_tiles < 0, problems or workspace NULL, a misaligned
 * or short workspace -> INVALID_VALUE; max_tiles above 2^24 - 1 ->
 * NOT_SUPPORTED; a failed launch -> LAUNCH.  num_groups == 0 or max_tiles ==
 * 0: nothing is enqueued (the workspace is not written). */
long long nvfp4_group_gemm_device_workspace_bytes(int num_groups); /* -1 if num_groups is out of range */
nvfp4_status nvfp4_group_gemm_device(const nvfp4_problem *problems, int num_groups, int max_tiles,
                                     void *workspace, long long workspace_bytes, hipStream_t stream);

/* ---- Blocked scale layout: the layout the kernelbot pages' kernels consume
 * (raw-CUDA page nvfp4-group-gemm-407526, device kernel, scale TMA issue: a
 * 128-row tile's scales start at (tile * K/64) * 512 bytes and advance 2048
 * bytes per 256 K; single-GEMM page nvfp4-gemm-125598, `custom_kernel`
 * docstring: permuted scales of shape [32, 4, rest_m, 4, rest_k, l]).
 *
 * 512-byte atoms, each holding the scales of 128 rows x 4 consecutive K/16
 * blocks; atom (row tile tm, K atom ka) at byte (tm * ceil(K/64) + ka) * 512;
 * inside it, row r (0..127) block c (0..3) at (r % 32) * 16 + (r / 32) * 4 +
 * c.  Rows pad to a multiple of 128 and blocks to a multiple of 4, with zero
 * bytes. */

/* Bytes of the blocked layout of a rows x K/16 scale matrix; -1 if rows < 0,
 * K < 0, K % 32 != 0 or K > 2^24. */
long long nvfp4_blocked_scale_bytes(int rows, int K);

/* Plain [rows][K/16] -> blocked (every byte of the blocked buffer is written,
 * padding as zero), and blocked -> plain.  Device pointers, the blocked one
 * 16-byte aligned; asynchronous on `stream`; rows == 0 or K == 0 does nothing.
 * Errors: INVALID_VALUE for negative sizes, NULL pointers (when there is
 * something to move) or a misaligned blocked pointer; NOT_SUPPORTED for
 * K % 32 != 0 or K > 2^24; LAUNCH if the kernel launch fails. */
nvfp4_status nvfp4_scales_to_blocked(const void *sf, void *blocked, int rows, int K,
                                     hipStream_t stream);
nvfp4_status nvfp4_scales_from_blocked(const void *blocked, void *sf, int rows, int K,
                                       hipStream_t stream);

/* nvfp4_gemm / nvfp4_group_gemm with SFA and SFB in the blocked layout
 * (16-byte aligned, nvfp4_blocked_scale_bytes(M or N, K) bytes each).  Where
 * the plain call would run the shared-decode 128 x 256 or 64 x 128 tiles
 * (large, grouped and large-N small-M products with every K % 256 == 0), the
 * 64 x 64 and 64 x 32 small-M tiles (every K % 256 == 0) or one-wave
 * 128 x 128 tiles (every K a multiple of 128), those kernels read the blocked
 * scales directly.  Otherwise (four waves per 128 x 128 tile, or K not a
 * multiple of those steps) the scales are first converted to the
 * plain layout inside the library's per-stream device workspace (so the call
 * may allocate it, and returns NOT_SUPPORTED inside a stream capture if it
 * would have to) and the plain path runs.  Either way C is bitwise what
 * nvfp4_gemm gives for the same scales.  Other arguments, limits and errors as
 * for the plain entry points. */
nvfp4_status nvfp4_gemm_blocked(const void *A, const void *SFA, const void *B, const void *SFB,
                                void *C, int M, int N, int K, hipStream_t stream);
nvfp4_status nvfp4_group_gemm_blocked(const nvfp4_problem *problems, int num_groups,
                                      hipStream_t stream);

/* ---- Power-of-two scales on the scaled FP4 MFMA.  Not a kernel of the
 * kernelbot pages: a special case of their operation (the grouped page
 * nvfp4-group-gemm-498453 and the single-GEMM page nvfp4-gemm-125598,
 * `custom_kernel`: C = A * SFA * B * SFB, sf_vec_size 16) for inputs whose
 * scales are all powers of two, which lets the packed e2m1 codes feed gfx950's
 * v_mfma_scale_f32_32x32x64_f8f6f4 without decoding (each scale becomes an
 * E8M0 exponent; each 16-value block rides in 32 MFMA K slots with 16 zeros).
 *
 * Same arguments, layouts, asynchrony and results as nvfp4_gemm /
 * nvfp4_group_gemm (fp32 accumulation, fp16 round-to-nearest-even), for
 * inputs whose every SFA and SFB code is a positive normal power of two:
 * e4m3fn codes 0x08, 0x10, ..., 0x78 (values 2^-6 .. 2^8).  Any other code
 * (nonzero mantissa, zero, subnormal, negative, NaN) is outside the contract:
 * its mantissa and sign bits are ignored, so C is wrong for it.  Each group
 * runs as one-wave 128 x 128 tiles over the whole of K (no K split, no
 * workspace).
 * Errors: as nvfp4_gemm / nvfp4_group_gemm, plus NOT_SUPPORTED when a
 * non-empty group has K % 128 != 0 or an SFA / SFB pointer that is not 8-byte
 * aligned. */
nvfp4_status nvfp4_gemm_pow2scale(const void *A, const void *SFA, const void *B, const void *SFB,
                                  void *C, int M, int N, int K, hipStream_t stream);
nvfp4_status nvfp4_group_gemm_pow2scale(const nvfp4_problem *problems, int num_groups,
                                        hipStream_t stream);

/* ---- Allocation-free single GEMM.  For callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, layouts, results (bitwise those of
 * nvfp4_gemm but for the one planning difference below) and errors as
 * nvfp4_gemm, with the same plan and kernels; the
 * calls that split K keep their tile counters and partial sums in a scratch
 * array of NVFP4_NOALLOC_SCRATCH_BYTES bytes that the library holds in device
 * memory on each GPU it runs on, until the process ends.  The call allocates
 * nothing (no hipMalloc, no library or torch allocation) and enqueues a small
 * kernel that clears the counters before the product, so it can be captured
 * on any stream.  One difference in planning: where nvfp4_gemm would split the
 * K of some 128 x 256 tiles for balance and their partial tiles would not fit
 * the array, this call keeps those tiles whole; C then differs from
 * nvfp4_gemm's only by fp32 summation order, within the same accuracy bound.
 * Every call on a GPU shares that GPU's array: calls that overlap in time on
 * one GPU (other streams, concurrent graph replays) race and give wrong
 * results.  The array holds no two-slice pair slots: two-slice sums take
 * the ticket protocol here, with bitwise the same results.  A plan whose
 * tile counters and partial sums would exceed the array
 * returns NVFP4_ERROR_NOT_SUPPORTED (the planner keeps the K-split launches
 * of small products at 256 workgroups of at most 32 KiB of partial sums,
 * within it). */
#define NVFP4_NOALLOC_SCRATCH_BYTES (16384 + 8388608)
nvfp4_status nvfp4_gemm_noalloc(const void *A, const void *SFA, const void *B, const void *SFB,
                                void *C, int M, int N, int K, hipStream_t stream);

/* How a call would be carried out (host only, no HIP call).  For tests and
 * reports. */
typedef struct {
    int kernel;      /* 0: nothing to launch, 1: one tile per workgroup, 2: K split
                        across workgroups, 3: a 128 x 128 tile's K split across
                        the workgroup's four waves, 4: four waves share a
                        128 x 256 tile (decoded A exchanged through LDS); the
                        tiles past whole rounds of one per CU may have their
                        K split across workgroups for balance; 5: eight waves
                        share a 64 x 128 tile (32 < M <= 64, at least 192
                        tiles) */
    int tile_m;      /* output rows per workgroup */
    int tile_n;      /* output columns per workgroup */
    int split_k;     /* K slices per output tile (1 = none; kernel 4: the
                        largest split of any tile) */
    int total_tiles; /* output tiles over all groups */
    int workgroups;  /* workgroups launched (kernels 1-3: total_tiles * split_k) */
    long long workspace_bytes; /* device workspace the call needs */
} nvfp4_plan_info;

/* Plan of nvfp4_gemm with these sizes; same argument rules (pointers are not
 * looked at).  `info` must not be NULL. */
nvfp4_status nvfp4_gemm_plan(int M, int N, int K, nvfp4_plan_info *info);

/* Plan of nvfp4_group_gemm.  `tile_prefix` (may be NULL) receives the
 * num_groups + 1 entries of the exclusive prefix over per-group tile counts. */
nvfp4_status nvfp4_group_gemm_plan(const nvfp4_problem *problems, int num_groups,
                                   nvfp4_plan_info *info, int *tile_prefix);

/* Frees every workspace the library holds (after synchronising its device).
 * Optional; for callers that want the memory back before process exit. */
nvfp4_status nvfp4_release_workspaces(void);

/* Static text for a status code. */
const char *nvfp4_status_string(nvfp4_status status);

/* NVFP4_ABI_VERSION of the built library. */
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
