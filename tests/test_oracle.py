"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each check is chosen so that a plausible slip in the oracle (a wrong table
entry, a swapped operand, a wrong scale index, a dropped term, a sign error,
a rounding mistake) fails at least one of them:
  * tables against the format definition (golden e2m1 table) and against an
    independent library decode (torch's float8_e4m3fn);
  * the binary16 rounding against numpy's double -> half conversion, ties and
    boundaries included;
  * closed forms (all ones gives K), special cases that reduce to a plain
    library matmul, scale linearity, sign and transpose symmetries, block
    permutation invariance;
  * exact rational brute force on tiny shapes.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from grouped_gemm_nvfp4_amd import inputs
from tests.parity import parity_failures, ulp16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden_e2m1():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return np.array([vals[c] for c in range(16)])


def torch_e4m3():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).double().numpy()


# ---------------------------------------------------------------- tables

def test_e2m1_table_matches_golden():
    t = oracle.e2m1_table()
    g = golden_e2m1()
    assert np.array_equal(t, g)
    assert np.array_equal(np.signbit(t), np.signbit(g))  # code 8 is -0


def test_e4m3_table_matches_library_decode():
    t = oracle.e4m3_table()
    ref = torch_e4m3()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    assert set(np.flatnonzero(np.isnan(t))) == {0x7F, 0xFF}
    fin = ~np.isnan(ref)
    assert np.array_equal(t[fin], ref[fin])


@pytest.mark.parametrize("code,value", [
    (0x7E, 448.0), (0xFE, -448.0), (0x01, 2.0 ** -9), (0x38, 1.0),
    (0x20, 0.125), (0x50, 8.0), (0x08, 2.0 ** -6), (0x07, 7 * 2.0 ** -9),
])
def test_e4m3_spot_values(code, value):
    assert oracle.e4m3_table()[code] == value


def test_scale_codes_of_recipe_are_the_range():
    t = oracle.e4m3_table()[inputs.SCALE_CODES]
    assert t.min() == 0.125 and t.max() == 8.0 and len(t) == 49
    assert np.all(np.diff(t) > 0)


def test_decode_low_nibble_is_even_k():
    # byte 0x71: low nibble code 1 (0.5) at k=0, high nibble code 7 (6.0) at k=1
    X = np.full((1, 8), 0x00, dtype=np.uint8)
    X[0, 0] = 0x71
    SF = np.array([[0x38]], dtype=np.uint8)
    d = oracle.decode(X, SF, 16)
    assert d[0, 0] == 0.5 and d[0, 1] == 6.0 and np.all(d[0, 2:] == 0)


def test_decode_scale_index_is_k_div_16():
    X = np.full((1, 16), 0x22, dtype=np.uint8)  # every element 1.0, K = 32
    SF = np.array([[0x40, 0x48]], dtype=np.uint8)  # 2.0 then 4.0
    d = oracle.decode(X, SF, 32)
    assert np.all(d[0, :16] == 2.0) and np.all(d[0, 16:] == 4.0)


# ---------------------------------------------------------------- fp16 rounding

def _numpy_half_bits(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def test_fp16_rne_random_against_numpy():
    rng = np.random.default_rng(7)
    mags = np.ldexp(rng.random(20000) + 0.5, rng.integers(-30, 18, 20000))
    x = mags * rng.choice([-1.0, 1.0], 20000)
    with np.errstate(over="ignore"):
        assert np.array_equal(oracle.fp16_rne(x), _numpy_half_bits(x))


def test_fp16_rne_ties_and_boundaries_against_numpy():
    pts = []
    # every tie midpoint between consecutive binary16 values in a few binades,
    # plus the subnormal range and the overflow threshold
    h = np.arange(0, 0x7C00, 37, dtype=np.uint16).view(np.float16).astype(np.float64)
    h1 = (np.arange(0, 0x7C00, 37, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    mids = (h + h1) / 2
    pts += list(mids) + list(np.nextafter(mids, 0)) + list(np.nextafter(mids, np.inf))
    pts += [0.0, -0.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -26,
            2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 65504.0, 65519.99, 65520.0,
            -65520.0, 1e9, 2047.5, 2048.5, 1.00048828125]
    x = np.array(pts)
    with np.errstate(over="ignore"):
        assert np.array_equal(oracle.fp16_rne(x), _numpy_half_bits(x))


def test_fp16_rne_nan():
    assert (int(oracle.fp16_rne(np.array([np.nan]))[0]) & 0x7FFF) > 0x7C00


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("K", [16, 256, 1536, 7168])
def test_all_ones_gives_K(K):
    M, N = 3, 5
    A = np.full((M, K // 2), 0x22, dtype=np.uint8)  # code 2 = 1.0 in both nibbles
    B = np.full((N, K // 2), 0x22, dtype=np.uint8)
    S1a = np.full((M, K // 16), 0x38, dtype=np.uint8)  # 1.0
    S1b = np.full((N, K // 16), 0x38, dtype=np.uint8)
    C16, C64, bound = oracle.gemm(A, S1a, B, S1b, M, N, K)
    assert np.all(C64 == K) and np.all(bound == K)
    assert np.all(C16.view(np.float16).astype(np.float64) == K)
    S2a = np.full((M, K // 16), 0x40, dtype=np.uint8)  # 2.0
    C16, C64, _ = oracle.gemm(A, S2a, B, S1b, M, N, K)
    assert np.all(C64 == 2 * K)


def test_group_gemm_each_group_its_own_closed_form():
    """Groups of different sizes, codes and scales: group g's product is its
    own closed form (all ones -> K; scales 2 x 2 -> 4K; code 0xA = -1.0 on one
    side -> -K), so a group computed with another group's sizes, buffers or
    scales fails; an empty group gives an empty result."""
    def ones(M, N, K, code_a=0x22, sa=0x38, sb=0x38):
        return {"A": np.full((M, K // 2), code_a, dtype=np.uint8),
                "SFA": np.full((M, K // 16), sa, dtype=np.uint8),
                "B": np.full((N, K // 2), 0x22, dtype=np.uint8),
                "SFB": np.full((N, K // 16), sb, dtype=np.uint8), "M": M, "N": N, "K": K}
    groups = [ones(3, 5, 256), ones(0, 4, 64), ones(2, 7, 1024, sa=0x40, sb=0x40),
              ones(6, 1, 96, code_a=0xAA)]
    expected = [256.0, None, 4 * 1024.0, -96.0]
    out = oracle.group_gemm(groups)
    assert len(out) == len(groups)
    for g, (C16, C64, bound), want in zip(groups, out, expected):
        assert C64.shape == (g["M"], g["N"])
        if want is None:
            continue
        assert np.all(C64 == want) and np.all(bound == abs(want))
        assert np.all(C16.view(np.float16).astype(np.float64) == want)


def test_overflow_rounds_to_infinity():
    K = 32
    A = np.full((2, K // 2), 0x77, dtype=np.uint8)  # 6.0
    A[1] = 0xFF                                      # -6.0
    B = np.full((1, K // 2), 0x77, dtype=np.uint8)
    SA = np.full((2, K // 16), 0x7E, dtype=np.uint8)  # 448
    SB = np.full((1, K // 16), 0x7E, dtype=np.uint8)
    C16, C64, _ = oracle.gemm(A, SA, B, SB, 2, 1, K)
    assert C16[0, 0] == 0x7C00 and C16[1, 0] == 0xFC00
    assert C64[0, 0] == K * (6 * 448.0) ** 2


# ------------------------------------------------ reductions to library routines

def _codes(X):
    """Unpacked codes [R][K] (low nibble = even k) -- test-side unpacking."""
    lo = X & 0xF
    hi = X >> 4
    return np.stack([lo, hi], axis=-1).reshape(X.shape[0], -1)


def test_unit_scales_reduce_to_library_matmul():
    rng = np.random.default_rng(11)
    M, N, K = 9, 7, 96
    p = inputs.draw_problem(rng, M, N, K)
    ones_a = np.full_like(p.SFA, 0x38)
    ones_b = np.full_like(p.SFB, 0x38)
    _, C64, bound = oracle.gemm(p.A, ones_a, p.B, ones_b, M, N, K)
    g = golden_e2m1()
    Ad, Bd = g[_codes(p.A)], g[_codes(p.B)]
    assert np.array_equal(C64, Ad @ Bd.T)
    assert np.array_equal(bound, np.abs(Ad) @ np.abs(Bd).T)


def test_unit_codes_reduce_to_scale_matmul():
    rng = np.random.default_rng(12)
    M, N, K = 6, 10, 128
    p = inputs.draw_problem(rng, M, N, K)
    A = np.full_like(p.A, 0x22)
    B = np.full_like(p.B, 0x22)
    _, C64, _ = oracle.gemm(A, p.SFA, B, p.SFB, M, N, K)
    t = torch_e4m3()
    SA, SB = t[p.SFA], t[p.SFB]
    assert np.array_equal(C64, 16.0 * (SA @ SB.T))


# ---------------------------------------------------------------- invariants

def test_scale_linearity_is_exact():
    rng = np.random.default_rng(13)
    M, N, K = 4, 6, 128
    p = inputs.draw_problem(rng, M, N, K)
    _, C64, _ = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    m, j = 2, 3
    SFA2 = p.SFA.copy()
    SFA2[m, j] += 8  # exponent + 1: the scale doubles (codes stay finite)
    assert oracle.e4m3_table()[SFA2[m, j]] == 2 * oracle.e4m3_table()[p.SFA[m, j]]
    _, C64b, _ = oracle.gemm(p.A, SFA2, p.B, p.SFB, M, N, K)
    # contribution of block j alone, from a 16-wide sub-problem
    blk = slice(8 * j, 8 * j + 8)
    _, Cj, _ = oracle.gemm(np.ascontiguousarray(p.A[:, blk]),
                           np.ascontiguousarray(p.SFA[:, j:j + 1]),
                           np.ascontiguousarray(p.B[:, blk]),
                           np.ascontiguousarray(p.SFB[:, j:j + 1]), M, N, 16)
    assert np.array_equal(C64b[m] - C64[m], Cj[m])
    others = [r for r in range(M) if r != m]
    assert np.array_equal(C64b[others], C64[others])


def test_sign_flip_negates():
    rng = np.random.default_rng(14)
    M, N, K = 5, 5, 64
    p = inputs.draw_problem(rng, M, N, K)
    _, C64, _ = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    _, C64n, _ = oracle.gemm(p.A ^ np.uint8(0x88), p.SFA, p.B, p.SFB, M, N, K)
    assert np.array_equal(C64n, -C64)


def test_operand_swap_transposes():
    rng = np.random.default_rng(15)
    M, N, K = 7, 3, 80
    p = inputs.draw_problem(rng, M, N, K)
    C16, C64, _ = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    C16t, C64t, _ = oracle.gemm(p.B, p.SFB, p.A, p.SFA, N, M, K)
    assert np.array_equal(C64t, C64.T) and np.array_equal(C16t, C16.T)


def test_block_permutation_invariance():
    rng = np.random.default_rng(16)
    M, N, K = 6, 8, 256
    p = inputs.draw_problem(rng, M, N, K)
    C16, C64, _ = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    perm = rng.permutation(K // 16)
    bperm = (perm[:, None] * 8 + np.arange(8)[None, :]).ravel()
    Ap = np.ascontiguousarray(p.A[:, bperm])
    Bp = np.ascontiguousarray(p.B[:, bperm])
    C16p, C64p, _ = oracle.gemm(Ap, np.ascontiguousarray(p.SFA[:, perm]), Bp,
                                np.ascontiguousarray(p.SFB[:, perm]), M, N, K)
    assert np.array_equal(C64p, C64) and np.array_equal(C16p, C16)


def test_entries_agree_with_full_product():
    rng = np.random.default_rng(17)
    M, N, K = 33, 29, 224
    p = inputs.draw_problem(rng, M, N, K)
    C16, C64, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    rows = rng.integers(0, M, 50)
    cols = rng.integers(0, N, 50)
    e16, e64, eb = oracle.gemm_entries(p.A, p.SFA, p.B, p.SFB, M, N, K, rows, cols)
    assert np.array_equal(e16, C16[rows, cols])
    assert np.array_equal(e64, C64[rows, cols])
    assert np.array_equal(eb, bound[rows, cols])


# ---------------------------------------------------------------- brute force

def _fraction_to_half_bits(q: Fraction) -> int:
    """binary16 RNE of an exact rational (independent of the oracle's routine)."""
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    if a == 0:
        return sign
    top = Fraction(65504) + Fraction(16)  # halfway to the next binade's first value
    if a >= top:
        return sign | 0x7C00
    e = -14
    while a >= Fraction(2) ** (e + 1) and e < 15:
        e += 1
    step = Fraction(2) ** (e - 10)  # spacing in this binade (also subnormals)
    n = a / step
    f = n.numerator // n.denominator
    rem = n - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    if a < Fraction(2) ** -14:
        return sign | f  # subnormal: f * 2^-24 (f == 1024 is the smallest normal)
    if f == 2048:
        f, e = 1024, e + 1
    if e > 15:
        return sign | 0x7C00
    return sign | ((e + 15) << 10) | (f - 1024)


def _frac_e4m3(c):
    s = -1 if c & 0x80 else 1
    e = (c >> 3) & 15
    m = c & 7
    if e == 0:
        return s * Fraction(m, 8) * Fraction(1, 64)
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def test_fraction_reference_rounding_self_check():
    # the test's own rational rounding agrees with numpy on exact binary values
    rng = np.random.default_rng(3)
    for v in np.ldexp(rng.random(300), rng.integers(-26, 17, 300)):
        assert _fraction_to_half_bits(Fraction(float(v))) == int(_numpy_half_bits(v))


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_exact_rationals(seed):
    rng = np.random.default_rng(100 + seed)
    M = int(rng.integers(1, 6))
    N = int(rng.integers(1, 6))
    K = int(rng.choice([16, 32, 48]))
    A = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    B = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    SFA = rng.choice(finite, (M, K // 16)).astype(np.uint8)
    SFB = rng.choice(finite, (N, K // 16)).astype(np.uint8)
    C16, C64, bound = oracle.gemm(A, SFA, B, SFB, M, N, K)
    e2 = [Fraction(float(v)) for v in golden_e2m1()]
    ca, cb = _codes(A), _codes(B)
    for m in range(M):
        for n in range(N):
            tot = Fraction(0)
            mag = Fraction(0)
            for k in range(K):
                t = (e2[ca[m, k]] * _frac_e4m3(int(SFA[m, k // 16]))
                     * e2[cb[n, k]] * _frac_e4m3(int(SFB[n, k // 16])))
                tot += t
                mag += abs(t)
            assert C64[m, n] == float(tot)
            assert bound[m, n] == float(mag)
            h = _fraction_to_half_bits(tot)
            if tot == 0:
                assert C16[m, n] & 0x7FFF == 0
            else:
                assert int(C16[m, n]) == h


def test_recipe_workload_is_exact_in_fp64():
    """Under the recipe's scale range every partial sum is a multiple of 2^-14
    below 2^26, so fp64 accumulation in any order is exact: the oracle's
    ascending loop and a library matmul agree bitwise."""
    rng = np.random.default_rng(18)
    M, N, K = 16, 12, 2048
    p = inputs.draw_problem(rng, M, N, K)
    _, C64, _ = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    g = golden_e2m1()
    t = torch_e4m3()
    Ad = g[_codes(p.A)] * np.repeat(t[p.SFA], 16, axis=1)
    Bd = g[_codes(p.B)] * np.repeat(t[p.SFB], 16, axis=1)
    assert np.array_equal(C64, Ad @ Bd.T)


# ---------------------------------------------------------------- parity rule

def test_parity_rule_accepts_and_rejects():
    ref = np.array([1.0, 1.0, 0.0, np.inf, 100.0], dtype=np.float16).view(np.uint16)
    bound = np.array([0.0, 0.0, 0.0, 1e9, 1000.0])
    ok = np.array([1.0 + 2 ** -10, 1.0, 0.0, np.inf, 100.9], dtype=np.float16).view(np.uint16)
    assert not parity_failures(ok, ref, bound).any()
    bad = np.array([1.0 + 2 ** -9, np.nan, 2 ** -23, -np.inf, 101.5],
                   dtype=np.float16).view(np.uint16)
    assert parity_failures(bad, ref, bound).all()
    assert ulp16(np.array([1.0]))[0] == 2.0 ** -10
    assert ulp16(np.array([0.0]))[0] == 2.0 ** -24
    assert ulp16(np.array([65504.0]))[0] == 32.0


# ------------------------------------------------------------ blocked scale layout

@pytest.mark.parametrize("rows,K", [(1, 32), (128, 256), (300, 96), (129, 1056), (512, 7168)])
def test_blocked_scales_round_trip(rows, K):
    rng = np.random.default_rng(rows + K)
    sf = rng.integers(0, 256, (rows, K // 16), dtype=np.uint8)
    blk = oracle.scales_to_blocked(sf, rows, K)
    assert blk.size == oracle.blocked_scale_shape(rows, K)[2]
    assert np.array_equal(oracle.scales_from_blocked(blk, rows, K), sf)
    # padding bytes are zero: exactly the non-padding bytes carry data
    assert np.count_nonzero(blk) == np.count_nonzero(sf)


def test_blocked_scales_follow_the_pages_atom_addressing():
    """The raw-CUDA page fetches, for 128-row tile t and 256-K step s, the 2048
    bytes at (t * K/64) * 512 + s * 2048: they must hold exactly the scales of
    rows [128 t, 128 t + 128) and blocks [16 s, 16 s + 16)."""
    rows, K = 384, 2048
    kb = K // 16
    # every (row, block) gets a 16-bit identity, carried through the byte
    # layout as two byte planes (no padding at this size)
    sf = np.arange(rows * kb, dtype=np.int64).reshape(rows, kb)
    lo = oracle.scales_to_blocked((sf & 0xFF).astype(np.uint8), rows, K).astype(np.int64)
    hi = oracle.scales_to_blocked((sf >> 8).astype(np.uint8), rows, K).astype(np.int64)
    ids = lo | (hi << 8)
    rest_k = K // 64
    for t in range(rows // 128):
        for s in range(K // 256):
            base = (t * rest_k) * 512 + s * 2048
            got = set(ids[base:base + 2048].tolist())
            want = {r * kb + j for r in range(128 * t, 128 * t + 128) for j in range(16 * s, 16 * s + 16)}
            assert got == want


def test_blocked_scales_row_within_atom():
    """Within one atom, rows r and r + 32 sit 4 bytes apart and rows r, r + 1
    sit 16 bytes apart ([32, 4, ..., 4, ...]: r % 32 outer, r // 32 next, the
    block innermost)."""
    rows, K = 128, 64
    sf = np.zeros((rows, 4), np.uint8)
    sf[33, 2] = 7          # r = 33: r % 32 = 1, r // 32 = 1, block 2
    blk = oracle.scales_to_blocked(sf, rows, K)
    assert np.flatnonzero(blk).tolist() == [1 * 16 + 1 * 4 + 2]


def test_blocked_scales_give_the_same_product():
    """C computed from scales that went through the blocked layout and back is
    bitwise the plain-layout C (the layout moves bytes only)."""
    from grouped_gemm_nvfp4_amd import inputs
    p = inputs.draw_problems(77, [(130, 70, 320)])[0]
    sfa = oracle.scales_from_blocked(oracle.scales_to_blocked(p.SFA, p.M, p.K), p.M, p.K)
    sfb = oracle.scales_from_blocked(oracle.scales_to_blocked(p.SFB, p.N, p.K), p.N, p.K)
    c1, _, _ = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
    c2, _, _ = oracle.gemm(p.A, sfa, p.B, sfb, p.M, p.N, p.K)
    assert np.array_equal(c1, c2)
