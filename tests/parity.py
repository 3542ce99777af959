"""Parity rule between a GPU result and the oracle.

Per element: |gpu - C16| <= 1e-3 * bound + ulp16(C16), where C16 is the
oracle's correctly rounded binary16 result, bound = sum_k |a_k * b_k| and
ulp16(x) is the binary16 spacing at |x| (2^-24 in the subnormal range).  When
C16 is an infinity the GPU value must be the same infinity; a NaN never passes.

The 1e-3 relative-to-bound term covers any fp32 accumulation order (an fp32
sum of K exact products is off by at most about K * 2^-24 * bound, far inside
it); the extra ulp covers the final rounding to binary16.
"""
from __future__ import annotations

import numpy as np

REL_TOL = 1e-3


def half_bits_to_f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def ulp16(x) -> np.ndarray:
    """binary16 spacing at |x| (finite x)."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.where(ax > 0, np.maximum(e, -14.0), -14.0)
    return np.ldexp(1.0, (e - 10).astype(np.int64))


def parity_failures(gpu_bits, ref_bits, bound) -> np.ndarray:
    """Boolean mask of elements that break the parity rule."""
    g = half_bits_to_f64(gpu_bits)
    r = half_bits_to_f64(ref_bits)
    bound = np.asarray(bound, dtype=np.float64)
    ref_inf = np.isinf(r)
    finite = ~ref_inf
    ok = np.zeros(r.shape, dtype=bool)
    ok[ref_inf] = g[ref_inf] == r[ref_inf]
    with np.errstate(invalid="ignore"):
        ok[finite] = (np.abs(g[finite] - r[finite])
                      <= REL_TOL * bound[finite] + ulp16(r[finite]))
    ok &= ~np.isnan(g)
    return ~ok


def assert_parity(gpu_bits, ref_bits, bound, what=""):
    bad = parity_failures(gpu_bits, ref_bits, bound)
    if bad.any():
        idx = np.argwhere(bad)
        first = tuple(int(i) for i in idx[0])
        g = half_bits_to_f64(gpu_bits)[first]
        r = half_bits_to_f64(ref_bits)[first]
        raise AssertionError(
            "%s: %d of %d elements break parity; first at %s: gpu=%r oracle=%r bound=%r"
            % (what, int(bad.sum()), bad.size, first, g, r,
               float(np.asarray(bound)[first])))
