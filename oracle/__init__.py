"""Plain CPU oracle for NVFP4 block-scaled GEMM and grouped GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU product path
(``grouped_gemm_nvfp4_amd``) never imports it, and the two share no code,
tables or constants; only the seeded input generator serves both.

The arithmetic lives in ``nvfp4_oracle.c`` (plain loops, fp64 accumulation,
a hand-written binary16 round-to-nearest-even).  This module builds it with
gcc, loads it with ctypes and hands numpy arrays across.

What is computed follows the kernelbot pages nvfp4-group-gemm-498453 and
nvfp4-gemm-125598 (``custom_kernel`` docstrings and the MMA loop, C = A * SFA *
B * SFB, one e4m3 scale per 16 K elements) and the grouped interface of
nvfp4-group-gemm-407526 (``group_gemm``: a list of independent problems, each
with its own M, N, K and buffers).

Every function is pinned in ``tests/test_oracle.py`` against closed forms,
an independent library decode, exact rational brute force, invariants and
special cases that reduce to a library matmul.  Nothing here is "parity
unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP) into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call([
            "gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
            "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm",
        ])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    lib.oracle_e2m1_value.argtypes = [ctypes.c_int]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [ctypes.c_int]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_fp16_rne.argtypes = [ctypes.c_double]
    lib.oracle_fp16_rne.restype = ctypes.c_uint16
    lib.oracle_decode_rows.argtypes = [u8p, u8p, ctypes.c_long, ctypes.c_long,
                                       ctypes.c_void_p]
    lib.oracle_decode_rows.restype = None
    lib.oracle_gemm.argtypes = [u8p, u8p, u8p, u8p, ctypes.c_long, ctypes.c_long,
                                ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_void_p]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_gemm_entries.argtypes = [u8p, u8p, u8p, u8p, ctypes.c_long,
                                        ctypes.c_long, ctypes.c_long, ctypes.c_long,
                                        ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.oracle_gemm_entries.restype = ctypes.c_int
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _u8(x: np.ndarray):
    assert x.dtype == np.uint8 and x.flags["C_CONTIGUOUS"], "packed operands are C-contiguous uint8"
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8))


def _ptr(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def e2m1_table() -> np.ndarray:
    """Value of each of the 16 e2m1 codes, from the format definition."""
    lib = _load()
    return np.array([lib.oracle_e2m1_value(c) for c in range(16)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    """Value of each of the 256 e4m3fn codes (NaN at 0x7F and 0xFF)."""
    lib = _load()
    return np.array([lib.oracle_e4m3_value(c) for c in range(256)], dtype=np.float64)


def fp16_rne(x) -> np.ndarray:
    """binary16 bit patterns (uint16) of doubles, round to nearest even."""
    lib = _load()
    flat = np.asarray(x, dtype=np.float64).ravel()
    out = np.fromiter((lib.oracle_fp16_rne(float(v)) for v in flat), dtype=np.uint16,
                      count=flat.size)
    return out.reshape(np.shape(x))


def decode(X: np.ndarray, SF: np.ndarray, K: int) -> np.ndarray:
    """Scaled fp64 values [R][K] of a packed operand X [R][K/2] with scales SF [R][K/16]."""
    lib = _load()
    R = X.shape[0]
    assert X.shape == (R, K // 2) and SF.shape == (R, K // 16)
    out = np.empty((R, K), dtype=np.float64)
    lib.oracle_decode_rows(_u8(X), _u8(SF), R, K, _ptr(out))
    return out


def gemm(A, SFA, B, SFB, M: int, N: int, K: int):
    """Full product: returns (C16 as uint16 bits, C64, bound), each [M][N]."""
    lib = _load()
    assert A.shape == (M, K // 2) and B.shape == (N, K // 2)
    assert SFA.shape == (M, K // 16) and SFB.shape == (N, K // 16)
    C16 = np.empty((M, N), dtype=np.uint16)
    C64 = np.empty((M, N), dtype=np.float64)
    bound = np.empty((M, N), dtype=np.float64)
    rc = lib.oracle_gemm(_u8(A), _u8(SFA), _u8(B), _u8(SFB), M, N, K,
                         _ptr(C16), _ptr(C64), _ptr(bound))
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments (rc=%d)" % rc)
    return C16, C64, bound


def gemm_entries(A, SFA, B, SFB, M: int, N: int, K: int, rows, cols):
    """Selected outputs (rows[i], cols[i]) computed one by one: (C16, C64, bound)."""
    lib = _load()
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.shape == cols.shape and rows.ndim == 1
    n = rows.size
    C16 = np.empty(n, dtype=np.uint16)
    C64 = np.empty(n, dtype=np.float64)
    bound = np.empty(n, dtype=np.float64)
    rc = lib.oracle_gemm_entries(_u8(A), _u8(SFA), _u8(B), _u8(SFB), M, N, K, n,
                                 _ptr(rows), _ptr(cols), _ptr(C16), _ptr(C64),
                                 _ptr(bound))
    if rc != 0:
        raise ValueError("oracle_gemm_entries rejected its arguments (rc=%d)" % rc)
    return C16, C64, bound


def group_gemm(problems):
    """Grouped product: ``problems`` is a list of dicts with keys A, SFA, B, SFB,
    M, N, K.  Each group is an independent product; returns a list of
    (C16, C64, bound)."""
    return [gemm(p["A"], p["SFA"], p["B"], p["SFB"], p["M"], p["N"], p["K"])
            for p in problems]


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return _load().oracle_num_threads()


# ---------------------------------------------------------------- blocked scales
#
# The scale layout the pages' kernels consume.  The raw-CUDA page
# (nvfp4-group-gemm-407526, device kernel, the scale TMA issue) addresses a
# 128-row tile's scales at (tile * K/64) * 512 bytes and advances 2048 bytes
# (four 512-byte atoms) per 256-element K step; the single-GEMM page
# (nvfp4-gemm-125598, `custom_kernel` docstring) gives the permuted scale
# tensor the shape [32, 4, rest_m, 4, rest_k, l].  Reading: one 512-byte atom
# holds the scales of 128 rows x 4 consecutive K/16 blocks, and within it the
# byte of row r (0..127) and block c (0..3) sits at (r % 32) * 16 + (r // 32)
# * 4 + c; atoms are ordered row tile major, K atom minor.  Rows are padded to
# a multiple of 128 and K/16 blocks to a multiple of 4 with zero bytes.


def blocked_scale_shape(rows: int, K: int):
    """(row tiles, K atoms, total bytes) of the blocked layout."""
    rest_m = (rows + 127) // 128
    rest_k = (K // 16 + 3) // 4
    return rest_m, rest_k, rest_m * rest_k * 512


def scales_to_blocked(sf: np.ndarray, rows: int, K: int) -> np.ndarray:
    """Plain [rows][K/16] scales -> the blocked byte layout (1-D uint8)."""
    rest_m, rest_k, _ = blocked_scale_shape(rows, K)
    kb = K // 16
    padded = np.zeros((rest_m * 128, rest_k * 4), np.uint8)
    padded[:rows, :kb] = np.asarray(sf, np.uint8).reshape(rows, kb)
    # [row tile, r // 32, r % 32, K atom, c] -> [row tile, K atom, r % 32, r // 32, c]
    t = padded.reshape(rest_m, 4, 32, rest_k, 4).transpose(0, 3, 2, 1, 4)
    return np.ascontiguousarray(t).reshape(-1)


def scales_from_blocked(blocked: np.ndarray, rows: int, K: int) -> np.ndarray:
    """The blocked byte layout -> plain [rows][K/16] scales."""
    rest_m, rest_k, nbytes = blocked_scale_shape(rows, K)
    t = np.asarray(blocked, np.uint8).reshape(-1)[:nbytes].reshape(rest_m, rest_k, 32, 4, 4)
    padded = t.transpose(0, 3, 2, 1, 4).reshape(rest_m * 128, rest_k * 4)
    return np.ascontiguousarray(padded[:rows, :K // 16])
