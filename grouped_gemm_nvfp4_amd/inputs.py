"""Seeded synthetic inputs for NVFP4 GEMM and grouped GEMM.

This module only draws random bytes; it holds none of the method's arithmetic
(no decoding, no products, no rounding).  Both the CPU oracle and the GPU path
consume what it returns.

Recipe (stated once, used everywhere):
  * ``rng = numpy.random.default_rng(seed)``; the named workloads below use
    ``seed = 1000 + index`` in the order they are listed.
  * Operands: e2m1 codes uniform over all 16 (both zeros included), drawn
    as a [rows][K] array and packed two per byte along K, the even K index
    in the low nibble: byte j of a row = code[2j] | code[2j + 1] << 4.
  * Scales: uniform over the 49 e4m3fn codes 0x20..0x50, the finite positive
    codes whose values lie in [0.125, 8].
  * Draw order, per group in order: A codes [M][K], B codes [N][K],
    SFA codes [M][K/16], SFB codes [N][K/16].  The 8-group MoE-like workload
    first draws its per-group M from {64, 128, ..., 512}.

These follow the leaderboard workloads the kernelbot pages were written for
(``custom_kernel`` docstrings: A [m, k/2] fp4 pairs, scales [m, k/16] e4m3,
C [m, n] fp16), whose own problem lists are not published.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np

# The 49 finite positive e4m3fn codes with values in [0.125, 8].
SCALE_CODES = np.arange(0x20, 0x51, dtype=np.uint8)
# Their powers of two (zero mantissa): 0.125, 0.25, ..., 8.
POW2_SCALE_CODES = np.arange(0x20, 0x51, 8, dtype=np.uint8)
GROUP_M_CHOICES = np.arange(64, 513, 64)


@dataclass
class Problem:
    """One independent product C[M][N] = A[M][K] . B[N][K]^T (packed, scaled)."""
    M: int
    N: int
    K: int
    A: np.ndarray    # uint8 [M][K/2]
    SFA: np.ndarray  # uint8 [M][K/16]
    B: np.ndarray    # uint8 [N][K/2]
    SFB: np.ndarray  # uint8 [N][K/16]

    def as_dict(self):
        return dict(M=self.M, N=self.N, K=self.K, A=self.A, SFA=self.SFA,
                    B=self.B, SFB=self.SFB)


def _packed_codes(rng: np.random.Generator, rows: int, K: int) -> np.ndarray:
    """rows x K uniform 4-bit codes, packed two per byte along K (even index
    in the low nibble): uint8 [rows][K/2]."""
    codes = rng.integers(0, 16, size=(rows, K), dtype=np.uint8)
    return np.ascontiguousarray(codes[:, 0::2] | (codes[:, 1::2] << 4))


def draw_problem(rng: np.random.Generator, M: int, N: int, K: int,
                 scale_codes: np.ndarray = SCALE_CODES) -> Problem:
    """Draw one problem's operands in the recipe's order."""
    if K % 16 != 0:
        raise ValueError("K must be a multiple of 16 (one scale per 16 elements)")
    A = _packed_codes(rng, M, K)
    B = _packed_codes(rng, N, K)
    SFA = rng.choice(scale_codes, size=(M, K // 16)).astype(np.uint8)
    SFB = rng.choice(scale_codes, size=(N, K // 16)).astype(np.uint8)
    return Problem(M, N, K, A, SFA, B, SFB)


def draw_problems(seed: int, shapes, scale_codes: np.ndarray = SCALE_CODES) -> List[Problem]:
    """Problems for a list of (M, N, K) shapes, drawn from one seeded stream
    (scales uniform over ``scale_codes``)."""
    rng = np.random.default_rng(seed)
    return [draw_problem(rng, M, N, K, scale_codes) for (M, N, K) in shapes]


@dataclass(frozen=True)
class Workload:
    name: str
    grouped: bool
    description: str


WORKLOADS = [
    Workload("gemm_128x128x256", False, "single GEMM M=128 N=128 K=256"),
    Workload("gemm_smallM_64x7168x16384", False,
             "small-M bandwidth-bound GEMM M=64 N=7168 K=16384"),
    Workload("gemm_large_8192x8192x8192", False,
             "large compute-bound GEMM M=N=K=8192"),
    Workload("group8_moe_N4096_K7168", True,
             "8 groups, M_g uniform in {64..512}, N=4096, K=7168"),
    Workload("group2_unequal", True,
             "2 groups (4096,3072,7168) + (384,3072,1536)"),
]


def workload_shapes(index: int):
    """(seed, [(M, N, K), ...]) of the named workload ``index``."""
    seed = 1000 + index
    if index == 0:
        return seed, [(128, 128, 256)]
    if index == 1:
        return seed, [(64, 7168, 16384)]
    if index == 2:
        return seed, [(8192, 8192, 8192)]
    if index == 3:
        rng = np.random.default_rng(seed)
        ms = rng.choice(GROUP_M_CHOICES, size=8)
        return seed, [(int(m), 4096, 7168) for m in ms]
    if index == 4:
        return seed, [(4096, 3072, 7168), (384, 3072, 1536)]
    raise IndexError(index)


def draw_workload(index: int, scale_codes: np.ndarray = SCALE_CODES) -> List[Problem]:
    """All problems of the named workload ``index`` (see ``WORKLOADS``), with
    scales uniform over ``scale_codes``.

    The 8-group workload's per-group M comes from the same seeded stream,
    drawn before the operands."""
    seed, shapes = workload_shapes(index)
    rng = np.random.default_rng(seed)
    if index == 3:
        rng.choice(GROUP_M_CHOICES, size=8)  # advance past the M draw
    return [draw_problem(rng, M, N, K, scale_codes) for (M, N, K) in shapes]


def flops(shapes) -> int:
    """Algorithmic work 2*M*N*K summed over problems."""
    return sum(2 * M * N * K for (M, N, K) in shapes)


def algorithmic_bytes(shapes) -> int:
    """Bytes the product must move at least once: packed A and B, their scales
    and the fp16 output."""
    return sum(M * K // 2 + N * K // 2 + M * K // 16 + N * K // 16 + 2 * M * N
               for (M, N, K) in shapes)
