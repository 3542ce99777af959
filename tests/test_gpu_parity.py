"""GPU parity: the gfx950 library against the CPU oracle, element by element.

Rule (tests/parity.py): |gpu - C16| <= 1e-3 * sum_k |a_k b_k| + ulp16(C16).
Every output buffer is poisoned with 0xFFFF (a NaN) before the call, so an
element the kernel fails to write shows up as a failure.  Small and medium
shapes and all five named workloads at full size are compared in full.  The
few shapes too large for a quick full oracle product are compared on sampled
outputs (whole rows and columns at the edges of the tiles the plan runs, the
last row and column always among them, plus random entries), which the
oracle computes one by one, and checked in full for unwritten elements.
"""
import numpy as np
import pytest

import oracle
from grouped_gemm_nvfp4_amd import inputs
from tests.parity import assert_parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import grouped_gemm_nvfp4_amd as g
    g.load()  # raises if the library is not built: no fallback
    return g


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def poisoned(M, N):
    return torch.full((M, N), -1, dtype=torch.int16, device="cuda")  # 0xFFFF


def dev_problem(p):
    return (to_dev(p.A), to_dev(p.SFA), to_dev(p.B), to_dev(p.SFB), poisoned(p.M, p.N))


def bits(C):
    return C.cpu().numpy().view(np.uint16)


def run_gemm(lib, p):
    A, SFA, B, SFB, C = dev_problem(p)
    lib.nvfp4_gemm(A, SFA, B, SFB, C, M=p.M, N=p.N, K=p.K)
    torch.cuda.synchronize()
    return bits(C)


def check_full(lib, p, what):
    got = run_gemm(lib, p)
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
    assert_parity(got, c16, bound, what)
    return got, c16


def edge_indices(L, tile):
    """Indices along one output dimension of length L where tile edges and
    masking act: the first and last index, the first index of the last tile,
    and both sides of every tile boundary."""
    s = {0, L - 1, ((L - 1) // tile) * tile}
    for e in range(tile - 1, L, tile):
        s |= {e, min(L - 1, e + 1)}
    return sorted(s)


def pick_edges(xs, n=12):
    """At most about n of the sorted edge indices: always the first two and
    the last three (the ragged tail), plus an even spread of the rest."""
    step = max(1, len(xs) // max(1, n - 5))
    return sorted(set(xs[:2] + xs[-3:] + xs[::step]))


def sample_positions(rng, M, N, tile_m=128, tile_n=128, n_random=3000):
    """Whole rows and whole columns at the tile edges of the plan that runs
    (first, last, the last tile's first, around internal boundaries), plus
    n_random random outputs."""
    rows, cols = [], []
    for r in pick_edges(edge_indices(M, tile_m)):
        rows += [r] * N
        cols += list(range(N))
    for c in pick_edges(edge_indices(N, tile_n)):
        rows += list(range(M))
        cols += [c] * M
    rows += list(rng.integers(0, M, n_random))
    cols += list(rng.integers(0, N, n_random))
    return np.array(rows), np.array(cols)


def plan_tile(lib, M, N, K):
    info = lib.gemm_plan(M, N, K)
    return info["tile_m"], info["tile_n"]


def check_sampled(got, p, seed, what, tile=(128, 128)):
    assert not np.any(got == 0xFFFF), "%s: unwritten (poisoned) outputs remain" % what
    rng = np.random.default_rng(seed)
    rows, cols = sample_positions(rng, p.M, p.N, tile[0], tile[1])
    c16, _, bound = oracle.gemm_entries(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K, rows, cols)
    assert_parity(got[rows, cols], c16, bound, what)


def check_against_full_oracle(got, p, what):
    """Every output against the oracle's full product (and none left
    unwritten: the poison is a NaN, which never passes)."""
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
    assert_parity(got, c16, bound, what)


# ------------------------------------------------------------------ single GEMM

def test_workload_128x128x256(lib):
    (p,) = inputs.draw_workload(0)
    check_full(lib, p, "128x128x256")


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 32), (17, 65, 64), (64, 64, 128), (65, 129, 96), (129, 200, 416),
    (200, 17, 256), (256, 384, 1024), (130, 260, 2080), (1, 300, 512), (300, 1, 160),
])
def test_edge_shapes(lib, M, N, K):
    p = inputs.draw_problems(2000 + M + 7 * N + K, [(M, N, K)])[0]
    check_full(lib, p, "edge %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [
    (64, 7168, 2080), (40, 1000, 1536), (64, 300, 16384), (1, 4097, 4096),
    (63, 257, 96), (33, 513, 8192), (64, 64, 16384), (5, 40, 9984),
])
def test_small_m_split_k_shapes(lib, M, N, K):
    """M <= 64 takes the stream kernel; few tiles make it split K as well."""
    info = lib.gemm_plan(M, N, K)
    assert info["tile_m"] == 64
    p = inputs.draw_problems(3000 + M + N + K, [(M, N, K)])[0]
    check_full(lib, p, "small-M %dx%dx%d split %d" % (M, N, K, info["split_k"]))


@pytest.mark.parametrize("M,N,K,kernel", [
    (1024, 65536, 128, 1),   # >= 4096 tiles: one wave per 128x128 tile
    (1800, 2000, 1184, 3),   # 240 tiles: four waves split each tile's K (ragged M, N and K)
])
def test_tiled_variants(lib, M, N, K, kernel):
    info = lib.gemm_plan(M, N, K)
    assert info["kernel"] == kernel and info["tile_m"] == 128
    p = inputs.draw_problems(4000 + M + K, [(M, N, K)])[0]
    if M * N <= 1 << 20:
        check_full(lib, p, "tiled %dx%dx%d" % (M, N, K))
    else:
        got = run_gemm(lib, p)
        check_sampled(got, p, 91, "tiled %dx%dx%d" % (M, N, K), plan_tile(lib, M, N, K))


@pytest.mark.parametrize("M,N,K", [
    (2300, 2170, 1024),  # K % 256 == 0: scales of two K tiles per load
    (2300, 2170, 1152),  # odd K tile count: per-K-tile scale loads
])
def test_one_wave_tiles_scale_loads(lib, M, N, K):
    """306 ragged one-wave 128 x 128 tiles, with each of the two ways the
    direct-to-LDS kernel fetches plain scales."""
    info = lib.gemm_plan(M, N, K)
    assert info["kernel"] == 1 and info["tile_m"] == 128
    p = inputs.draw_problems(4100 + K, [(M, N, K)])[0]
    got = run_gemm(lib, p)
    check_sampled(got, p, 4101 + K, "one-wave %dx%dx%d" % (M, N, K), plan_tile(lib, M, N, K))


@pytest.mark.parametrize("M,N,K", [
    (2048, 2048, 512),   # two of the four waves get no K tile (zero partial tiles)
    (1700, 1900, 2048),  # ragged M and N, scales two K tiles per load
    (2027, 1839, 1536),  # six pairs of K tiles: quarters of 1, 2, 1 and 2 pairs
    (1800, 2000, 1152),  # odd K tile count: per-K-tile scale loads
])
def test_four_wave_direct_tiles(lib, M, N, K):
    """The four-wave form of the direct-to-LDS 128 x 128 tile: each wave takes
    a quarter of K in its own LDS region, the partial tiles are added through
    LDS and wave 0 writes C."""
    info = lib.gemm_plan(M, N, K)
    assert info["kernel"] == 3 and info["tile_m"] == 128
    p = inputs.draw_problems(4200 + K, [(M, N, K)])[0]
    got = run_gemm(lib, p)
    check_sampled(got, p, 4201 + K, "four-wave %dx%dx%d" % (M, N, K), plan_tile(lib, M, N, K))
    assert np.array_equal(got, run_gemm(lib, p)), "four-wave sums must not depend on timing"


@pytest.mark.parametrize("M,N,K,split", [
    (48, 12288, 4128, 1),   # K % 256 != 0: byte scale loads, ragged last K tile
    (64, 6400, 8224, 2),    # byte scale loads with a K split
    (63, 7000, 4640, 2),    # ragged M and N, K % 256 != 0
])
def test_panel_shapes(lib, M, N, K, split):
    """M <= 64 with enough 64 x 64 tiles (and K slices) to fill the chip, and
    K % 256 != 0 (outside the 64 x 128 tile's contract), takes the panel
    kernel."""
    info = lib.gemm_plan(M, N, K)
    assert info["tile_n"] == 64 and info["split_k"] == split
    p = inputs.draw_problems(5000 + M + K, [(M, N, K)])[0]
    check_full(lib, p, "panel %dx%dx%d split %d" % (M, N, K, split))


@pytest.mark.parametrize("M,N,K,tile_n,split", [
    (64, 28672, 4096, 128, 1),  # 224 tiles of 64 x 128: two column waves share decoded A
    (40, 24576, 2048, 128, 1),  # 192 tiles, ragged M, one pair of K tiles per K-group
    (33, 30000, 1280, 128, 1),  # ragged M and N, 5 pairs: K-groups of 2, 2, 1 and 0 pairs
    (64, 6144, 8192, 64, 2),    # too few 64 x 128 tiles: the panel kernel
])
def test_small_m_wide_tile_shapes(lib, M, N, K, tile_n, split):
    """32 < M <= 64 with every K % 256 == 0 and at least 192 tiles of 64 x 128
    takes the 64 x 128 tile of the direct-to-LDS pipeline (four K-groups of two
    waves sharing their decoded A rows); with fewer, the panel kernel."""
    info = lib.gemm_plan(M, N, K)
    assert info["kernel"] == (5 if tile_n == 128 else 2) and (info["tile_m"], info["tile_n"]) == (64, tile_n)
    assert info["split_k"] == split
    p = inputs.draw_problems(5400 + M + K, [(M, N, K)])[0]
    got = run_gemm(lib, p)
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    assert_parity(got, c16, bound, "small-M wide %dx%dx%d split %d" % (M, N, K, split))
    assert np.array_equal(got, run_gemm(lib, p)), "the K-group and slice sums must not depend on timing"


@pytest.mark.parametrize("M,N,K", [(64, 6144, 8192), (40, 500, 1024), (200, 136, 512)])
def test_scale_pointers_at_odd_offsets(lib, M, N, K):
    """Scale arrays that start at an odd byte address take the byte-load
    paths of every kernel."""
    p = inputs.draw_problems(5100 + M, [(M, N, K)])[0]
    A, _, B, _, C = dev_problem(p)
    sfa = torch.zeros(p.SFA.size + 1, dtype=torch.uint8, device="cuda")
    sfb = torch.zeros(p.SFB.size + 1, dtype=torch.uint8, device="cuda")
    sfa[1:] = to_dev(p.SFA.reshape(-1))
    sfb[1:] = to_dev(p.SFB.reshape(-1))
    assert sfa[1:].data_ptr() % 2 == 1
    lib.nvfp4_gemm(A, sfa[1:], B, sfb[1:], C, M=M, N=N, K=K)
    torch.cuda.synchronize()
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    assert_parity(bits(C), c16, bound, "odd scale pointers %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [
    (128, 128, 256),     # one 128 x 128 tile: eight 64 x 32 tiles
    (512, 512, 16384),   # 16 tiles of 128 x 128: 64 x 64 tiles, K split in four
    (300, 520, 16384),   # ragged M and N, K split in five
    (129, 257, 32768),   # mostly padding rows and columns, K split in sixteen
])
def test_few_tiles_take_64_row_kernels(lib, M, N, K):
    """M > 64 with at most 128 tiles of 128 x 128 runs on the 64-row kernels
    (eight waves per workgroup, K split within and across workgroups)."""
    info = lib.gemm_plan(M, N, K)
    assert info["tile_m"] == 64
    p = inputs.draw_problems(5200 + M + K, [(M, N, K)])[0]
    check_full(lib, p, "few tiles %dx%dx%d split %d" % (M, N, K, info["split_k"]))


def _random_regime_shapes():
    rng = np.random.default_rng(2024)
    shapes = []
    for regime in range(6):
        for _ in range(2):
            if regime == 0:    # M <= 64
                shapes.append((int(rng.integers(1, 65)), int(rng.integers(1, 9000)), 32 * int(rng.integers(1, 400))))
            elif regime == 1:  # M > 64, few 128 x 128 tiles: 64-row kernels
                shapes.append((int(rng.integers(65, 1600)), int(rng.integers(1, 1600)), 32 * int(rng.integers(1, 300))))
            elif regime == 2:  # many tiles, K % 128 == 0
                shapes.append((int(rng.integers(1000, 4200)), int(rng.integers(1000, 4200)), 128 * int(rng.integers(1, 24))))
            elif regime == 3:  # many tiles, K % 256 == 0 (scales two K tiles per load)
                shapes.append((int(rng.integers(1500, 3500)), int(rng.integers(1500, 3500)), 256 * int(rng.integers(1, 12))))
            elif regime == 4:  # the 128 x 256 wide tile, its balancing split and M-edge tiles
                shapes.append((int(rng.integers(2048, 5000)), int(rng.integers(2048, 5000)), 256 * int(rng.integers(1, 16))))
            else:              # 32 < M <= 64 with many columns: the 64 x 128 small-M tile
                shapes.append((int(rng.integers(33, 65)), int(rng.integers(24600, 40000)), 256 * int(rng.integers(2, 16))))
    return shapes


@pytest.mark.parametrize("M,N,K", _random_regime_shapes())
def test_random_shapes_across_planner_regimes(lib, M, N, K):
    """Seeded random shapes in each of the planner's regimes; outputs checked
    in full where the oracle is quick, else sampled (edge rows and columns
    included), and never left unwritten."""
    p = inputs.draw_problems(9100 + M + K, [(M, N, K)])[0]
    if M * N <= 300_000:
        check_full(lib, p, "random %dx%dx%d" % (M, N, K))
    else:
        check_sampled(run_gemm(lib, p), p, 9101 + N, "random %dx%dx%d" % (M, N, K), plan_tile(lib, M, N, K))


def _random_moe_groups():
    """Seeded mixture-of-experts-like group lists: ragged row counts (M-edge
    tiles of every kind), one N and K per list, enough 128 x 256 tiles for
    the wide route."""
    rng = np.random.default_rng(2025)
    cases = []
    for _ in range(3):
        G = int(rng.integers(5, 11))
        N = int(rng.choice([2048, 3072, 4096]))
        K = 256 * int(rng.integers(4, 24))
        cases.append([(int(rng.integers(1, 700)), N, K) for _ in range(G)])
    return cases


@pytest.mark.parametrize("case", range(3))
def test_random_moe_groups_on_the_wide_tile(lib, case):
    """Random MoE-like grouped launches on the 128 x 256 tile: striped tile
    orders, M-edge tiles with one to three live row blocks, and the balancing
    split, every group checked against the oracle."""
    shapes = _random_moe_groups()[case]
    info, _ = lib.group_gemm_plan(shapes)
    while info["kernel"] != 4:   # grow every group until the launch has 256 wide tiles
        shapes = [(M + 128, N, K) for (M, N, K) in shapes]
        info, _ = lib.group_gemm_plan(shapes)
    assert info["kernel"] == 4
    probs = inputs.draw_problems(9300 + case, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        if p.M * p.N <= 1_000_000:
            c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
            assert_parity(got, c16, bound, "moe case %d group %d" % (case, i))
        else:
            check_sampled(got, p, 9310 + i, "moe case %d group %d" % (case, i), (128, 256))


def test_few_tiles_deterministic(lib):
    """The last arriver adds the K slices in slice order, so repeated calls
    agree bit for bit whatever order the workgroups finish in."""
    p = inputs.draw_problems(5300, [(512, 512, 16384)])[0]
    runs = [run_gemm(lib, p) for _ in range(3)]
    assert np.array_equal(runs[0], runs[1]) and np.array_equal(runs[0], runs[2])


def test_all_ones_gives_exactly_K(lib):
    M, N, K = 130, 70, 7168
    ones = inputs.Problem(M, N, K, np.full((M, K // 2), 0x22, np.uint8),
                          np.full((M, K // 16), 0x38, np.uint8),
                          np.full((N, K // 2), 0x22, np.uint8),
                          np.full((N, K // 16), 0x38, np.uint8))
    got = run_gemm(lib, ones)
    assert np.all(got.view(np.float16) == np.float16(K))


def test_exhaustive_decode_table(lib):
    """All 16 e2m1 codes x all 254 finite e4m3 scales through the GEMM path:
    row (c, s) holds code c at k = 0 with scale s; B is 1.0 at k = 0 with unit
    scale, so C = e2m1(c) * e4m3(s), exact in fp16."""
    K = 32
    scales = [s for s in range(256) if (s & 0x7F) != 0x7F]
    M = 16 * len(scales)
    A = np.zeros((M, K // 2), np.uint8)
    SFA = np.zeros((M, K // 16), np.uint8)
    for i, (c, s) in enumerate((c, s) for c in range(16) for s in scales):
        A[i, 0] = c
        SFA[i, 0] = s
    B = np.zeros((1, K // 2), np.uint8)
    B[0, 0] = 0x02
    SFB = np.full((1, K // 16), 0x38, np.uint8)
    p = inputs.Problem(M, 1, K, A, SFA, B, SFB)
    got, c16 = check_full(lib, p, "decode table")
    # exact: every product e2m1 * e4m3 is representable in fp16
    nz = (c16 & 0x7FFF) != 0
    assert np.array_equal(got[nz], c16[nz])


def test_k_zero_fills_zero(lib):
    C = poisoned(33, 47)
    lib.nvfp4_gemm(None, None, None, None, C, M=33, N=47, K=0)
    torch.cuda.synchronize()
    assert np.all(bits(C) == 0)


def test_empty_output_is_noop(lib):
    C = poisoned(4, 4)
    lib.nvfp4_gemm(None, None, None, None, C, M=0, N=4, K=64)
    lib.nvfp4_gemm(None, None, None, None, C, M=4, N=0, K=64)
    torch.cuda.synchronize()
    assert np.all(bits(C) == 0xFFFF)


def test_deterministic(lib):
    p = inputs.draw_problems(77, [(300, 520, 3072)])[0]
    a = run_gemm(lib, p)
    b = run_gemm(lib, p)
    assert np.array_equal(a, b)


def test_overflow_gives_infinity(lib):
    M, N, K = 2, 3, 64
    A = np.full((M, K // 2), 0x77, np.uint8)
    A[1] = 0xFF
    B = np.full((N, K // 2), 0x77, np.uint8)
    SA = np.full((M, K // 16), 0x7E, np.uint8)
    SB = np.full((N, K // 16), 0x7E, np.uint8)
    p = inputs.Problem(M, N, K, A, SA, B, SB)
    got, _ = check_full(lib, p, "overflow")
    assert np.all(got[0] == 0x7C00) and np.all(got[1] == 0xFC00)


@pytest.mark.parametrize("index", [1, 2])
def test_full_size_single_workloads(lib, index):
    """The small-M (64 x 7168 x 16384) and large (8192^3) workloads at full
    size, in the launch configuration bench.py times, every output against the
    oracle's full product."""
    (p,) = inputs.draw_workload(index)
    got = run_gemm(lib, p)
    check_against_full_oracle(got, p, inputs.WORKLOADS[index].name)


@pytest.mark.parametrize("M,N,kernel_tile", [
    (4, 64, 64),       # 64-row kernels: K split across eight waves and the workgroups
    (256, 16512, 128), # 258 one-wave 128 x 128 tiles: one serial chain over all of K
])
def test_largest_k_all_positive(lib, M, N, kernel_tile):
    """K at the library's limit (NVFP4_MAX_K = 131072) with every term
    positive, so every partial sum is as large as the final one: the case where
    fp32 rounding, relative to the bound sum_k |a_k b_k|, is largest.  The
    parity tolerance must still hold there."""
    K = 131072
    info = lib.gemm_plan(M, N, K)
    assert info["tile_m"] == kernel_tile
    rng = np.random.default_rng(6000 + M)
    p = inputs.draw_problems(6000 + M, [(M, N, K)])[0]
    # positive e2m1 codes only: clear the sign bit of both nibbles
    p.A &= 0x77
    p.B &= 0x77
    got = run_gemm(lib, p)
    if M * N <= 1 << 16:
        check_against_full_oracle(got, p, "K=%d all positive %dx%d" % (K, M, N))
    else:
        check_sampled(got, p, int(rng.integers(1 << 30)), "K=%d all positive %dx%d" % (K, M, N),
                      plan_tile(lib, M, N, K))


# ------------------------------------------------- two-slice pair slots

def test_two_slice_pairs_across_interleaved_calls(lib):
    """Two-slice K splits on the 64 x 64 panel tile sum their slices through
    the workspace's pair slots, which every such call must leave at their
    empty state.  On one stream: a two-slice panel call, a two-slice stream
    call (ticket protocol), a wide-tile call whose K split uses the partial
    tiles after the pair slots, the same two-slice calls again on new data,
    a two-slice panel call whose slices run on different XCDs, and a
    two-slice grouped panel call; each against the oracle, and the
    repeated calls bitwise equal to the allocation-free entry point's sums
    (which keeps no pair slots and takes the ticket protocol)."""
    panel, stream_, wide = (100, 3072, 4096), (33, 2400, 2048), (2304, 4096, 1024)
    # 98 tiles, 196 workgroups: not a multiple of the eight XCDs, so the two
    # slices of a tile run on neighbouring XCDs (the pairs meet across L2s)
    cross = (100, 3104, 4096)
    for shape, tile_n in ((panel, 64), (cross, 64), (stream_, 32)):
        info = lib.gemm_plan(*shape)
        assert (info["tile_n"], info["split_k"]) == (tile_n, 2), shape
    assert lib.gemm_plan(*cross)["workgroups"] % 8 != 0
    info = lib.gemm_plan(*wide)
    assert info["kernel"] == 4 and info["split_k"] > 1
    seq = [panel, stream_, wide, panel, stream_, cross]
    probs = inputs.draw_problems(7700, seq)
    outs = []
    for p in probs:
        A, SFA, B, SFB, C = dev_problem(p)
        lib.nvfp4_gemm(A, SFA, B, SFB, C, M=p.M, N=p.N, K=p.K)
        outs.append((C, (A, SFA, B, SFB)))
    torch.cuda.synchronize()
    for i, (p, (C, _)) in enumerate(zip(probs, outs)):
        what = "call %d %dx%dx%d" % (i, p.M, p.N, p.K)
        if p.M * p.N <= 400_000:
            check_against_full_oracle(bits(C), p, what)
        else:
            check_sampled(bits(C), p, 7701 + i, what, plan_tile(lib, p.M, p.N, p.K))
    for i in (3, 4, 5):
        p = probs[i]
        A, SFA, B, SFB = outs[i][1]
        C2 = poisoned(p.M, p.N)
        lib.nvfp4_gemm_noalloc(A, SFA, B, SFB, C2, M=p.M, N=p.N, K=p.K)
        torch.cuda.synchronize()
        assert np.array_equal(bits(C2), bits(outs[i][0])), "pair and ticket sums differ, call %d" % i
    group = [(80, 2048, 4096), (40, 2048, 4096), (3, 256, 4096)]
    ginfo, _ = lib.group_gemm_plan(group)
    assert (ginfo["tile_n"], ginfo["split_k"]) == (64, 2)
    gprobs = inputs.draw_problems(7710, group)
    for i, (p, got) in enumerate(zip(gprobs, run_group(lib, gprobs))):
        check_against_full_oracle(got, p, "two-slice group %d" % i)


@pytest.mark.parametrize("M,N,K", [
    (100, 3071, 4096),   # odd N: two-byte stores, the last pair's second column past N
    (20, 7167, 16384),   # M <= 32 (one row block) and odd N
    (1, 7001, 16384),    # a single row; 220 workgroups, not a multiple of 8
])
def test_two_slice_pairs_ragged_edges(lib, M, N, K):
    """Two-slice panel launches at ragged edges: every output against the
    oracle and bitwise the allocation-free entry point's ticket sums."""
    info = lib.gemm_plan(M, N, K)
    assert (info["tile_n"], info["split_k"]) == (64, 2)
    p = inputs.draw_problems(7740 + M, [(M, N, K)])[0]
    A, SFA, B, SFB, C = dev_problem(p)
    lib.nvfp4_gemm(A, SFA, B, SFB, C, M=M, N=N, K=K)
    torch.cuda.synchronize()
    got = bits(C)
    check_against_full_oracle(got, p, "two-slice %dx%dx%d" % (M, N, K))
    C2 = poisoned(M, N)
    lib.nvfp4_gemm_noalloc(A, SFA, B, SFB, C2, M=M, N=N, K=K)
    torch.cuda.synchronize()
    assert np.array_equal(bits(C2), got), "pair and ticket sums differ"


@pytest.mark.parametrize("M,N,K,split", [
    (64, 7168, 4096, 2),    # one K tile per wave: each wave's trip ends after one step
    (24, 7168, 8192, 2),    # the one-row-block form, two tiles per wave
    (17, 4096, 12800, 4),   # 50 K tiles in four slices of 12 or 13: uneven trips, ticket sums
    (48, 7000, 6016, 2),    # K % 256 != 0: byte-wise scales, a ragged last K tile
])
def test_panel_tail_form(lib, M, N, K, split):
    """Panel launches whose waves' K-tile counts are not multiples of four
    take the form that stops each wave's last trip at its last tile: every
    output against the oracle, and (K % 256 == 0) blocked scales bitwise the
    plain call."""
    info = lib.gemm_plan(M, N, K)
    nkt = (K + 255) // 256
    assert (info["tile_n"], info["split_k"]) == (64, split)
    assert nkt % split != 0 or (nkt // split) % 32 != 0
    p = inputs.draw_problems(7750 + M, [(M, N, K)])[0]
    A, SFA, B, SFB, C = dev_problem(p)
    lib.nvfp4_gemm(A, SFA, B, SFB, C, M=M, N=N, K=K)
    torch.cuda.synchronize()
    got = bits(C)
    check_against_full_oracle(got, p, "panel tail %dx%dx%d" % (M, N, K))
    if K % 256 == 0:
        C2 = poisoned(M, N)
        lib.nvfp4_gemm_blocked(A, blocked_dev(p.SFA, M, K), B, blocked_dev(p.SFB, N, K), C2, M, N, K)
        torch.cuda.synchronize()
        assert np.array_equal(bits(C2), got), "blocked scales change C"


def test_two_slice_pairs_repeat_bitwise(lib):
    """Twelve calls alternating two two-slice panel products (one with its
    slices on different XCDs) and a ticket-summed stream product on one
    stream, C poisoned before each: the first call of each product matches
    the oracle, and every later call's C is bitwise the first call's (the pair
    slots return to their empty state after every launch, whatever ran
    before)."""
    shapes = [(64, 7168, 16384), (100, 3104, 4096), (33, 2400, 2048)]
    probs = inputs.draw_problems(7720, shapes)
    devs = [dev_problem(p) for p in probs]
    first = [None] * len(shapes)
    for call in range(12):
        i = call % len(shapes)
        p, (A, SFA, B, SFB, C) = probs[i], devs[i]
        C.fill_(-1)
        lib.nvfp4_gemm(A, SFA, B, SFB, C, M=p.M, N=p.N, K=p.K)
        torch.cuda.synchronize()
        got = bits(C)
        if first[i] is None:
            check_against_full_oracle(got, p, "first call %dx%dx%d" % (p.M, p.N, p.K))
            first[i] = got
        else:
            assert np.array_equal(got, first[i]), "call %d differs, %dx%dx%d" % (call, p.M, p.N, p.K)


HIP_STREAM_PER_THREAD = 2  # hipStreamPerThread in hip_runtime_api.h


@pytest.mark.parametrize("streams", ["own", "per-thread"])
def test_concurrent_streams_keep_their_own_workspaces(lib, streams):
    """Two host threads issue K-split calls at the same time, each on a
    stream of its own (a torch stream each, or hipStreamPerThread, which names
    a different stream in every thread): two-slice panel calls (pair slots), a
    ticket-summed stream call and a wide-tile balancing split.  Every output
    is bitwise the one a serial run on the default stream gives, so the two
    streams never share tile counters, pair slots or partial tiles."""
    import threading
    from grouped_gemm_nvfp4_amd import _binding as b
    shapes = [(100, 3072, 4096), (64, 7168, 16384), (64, 1024, 8192), (2304, 4096, 1024)]
    splits = [lib.gemm_plan(*sh)["split_k"] for sh in shapes]
    assert splits[0] == 2 and splits[1] == 2 and min(splits) > 1
    probs = inputs.draw_problems(7730, shapes)
    devs = [dev_problem(p) for p in probs]
    ref = []
    for p, (A, SFA, B, SFB, C) in zip(probs, devs):
        lib.nvfp4_gemm(A, SFA, B, SFB, C, M=p.M, N=p.N, K=p.K)
        torch.cuda.synchronize()
        ref.append(bits(C))
    iters = 3
    outs = [[[poisoned(p.M, p.N) for p in probs] for _ in range(iters)] for _ in range(2)]
    torch_streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    errors = []

    def work(t):
        try:
            handle = HIP_STREAM_PER_THREAD if streams == "per-thread" else torch_streams[t].cuda_stream
            for it in range(iters):
                for p, (A, SFA, B, SFB, _), C in zip(probs, devs, outs[t][it]):
                    rc = b.raw_gemm(A.data_ptr(), SFA.data_ptr(), B.data_ptr(), SFB.data_ptr(), C.data_ptr(),
                                    p.M, p.N, p.K, handle)
                    if rc != b.NVFP4_OK:
                        errors.append((t, it, rc))
        except Exception as e:  # reported below, on the main thread
            errors.append((t, repr(e)))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t in range(2):
        for it in range(iters):
            for i, p in enumerate(probs):
                assert np.array_equal(bits(outs[t][it][i]), ref[i]), \
                    "thread %d call %d %dx%dx%d differs" % (t, it, p.M, p.N, p.K)


# ------------------------------------------------------------------ grouped GEMM

def run_group(lib, probs):
    devs = [dev_problem(p) for p in probs]
    lib.nvfp4_group_gemm([d + (p.M, p.N, p.K) for d, p in zip(devs, probs)])
    torch.cuda.synchronize()
    return [bits(d[4]) for d in devs]


def test_group_small_full_compare(lib):
    shapes = [(64, 256, 512), (0, 128, 256), (200, 130, 256), (1, 1, 32), (128, 0, 64),
              (129, 257, 1536), (64, 256, 512)]
    probs = inputs.draw_problems(31, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        if p.M == 0 or p.N == 0:
            continue
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "group %d" % i)


def test_group_small_m_split_k(lib):
    rng = np.random.default_rng(36)
    shapes = [(int(rng.integers(1, 65)), int(rng.integers(1, 200)), 32 * int(rng.integers(64, 160)))
              for _ in range(4)] + [(0, 64, 64), (64, 64, 0), (7, 33, 96)]
    info, _ = lib.group_gemm_plan(shapes)
    assert info["split_k"] > 1
    probs = inputs.draw_problems(37, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        if p.M == 0 or p.N == 0:
            continue
        if p.K == 0:
            assert np.all(got == 0)
            continue
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "small-M group %d" % i)


@pytest.mark.parametrize("M,N,K,split", [
    (1, 7168, 16384, 2),    # one row, scale groups of four K tiles
    (32, 6144, 8192, 2),    # exactly one 32-row block
    (17, 12288, 4128, 1),   # K % 256 != 0: byte scale loads, ragged last K tile
    (32, 6400, 8224, 2),    # byte scale loads with a K split
    (31, 7000, 8192, 2),    # ragged M and N
])
def test_panel_one_row_block(lib, M, N, K, split):
    """M <= 32 on the panel kernel: only rows 0..31 of A are loaded and
    decoded, two MFMAs per step."""
    info = lib.gemm_plan(M, N, K)
    assert info["tile_n"] == 64 and info["split_k"] == split
    p = inputs.draw_problems(5100 + M + K, [(M, N, K)])[0]
    check_full(lib, p, "panel one block %dx%dx%d split %d" % (M, N, K, split))


def test_group_panel_one_row_block(lib):
    """A grouped panel launch whose groups all have M <= 32."""
    shapes = [(32, 2048, 8192), (1, 2000, 8192), (20, 2048, 4096), (9, 1900, 8192)]
    info, _ = lib.group_gemm_plan(shapes)
    assert info["tile_n"] == 64 and info["split_k"] > 1
    probs = inputs.draw_problems(39, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "panel one-block group %d" % i)


def test_group_small_m_panel(lib):
    """Small-M groups whose 64 x 64 tiles fill the chip take the panel kernel
    with a K split (one K % 256 != 0); ragged N and M in some groups."""
    shapes = [(64, 2048, 8192), (17, 2000, 8192), (64, 2048, 4128), (50, 1900, 8192)]
    info, _ = lib.group_gemm_plan(shapes)
    assert info["tile_n"] == 64 and info["split_k"] > 1
    probs = inputs.draw_problems(38, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "panel group %d" % i)


def test_group_few_tiles_mixed(lib):
    """A grouped launch with few 128 x 128 tiles on the 64-row kernels: ragged
    M and N above 64, different K per group, a K = 0 group (zero C) and an
    empty group."""
    shapes = [(300, 400, 8192), (129, 257, 16384), (200, 100, 0), (0, 64, 256), (256, 384, 8192), (65, 700, 6144)]
    info, _ = lib.group_gemm_plan(shapes)
    assert info["tile_m"] == 64 and info["split_k"] > 1
    probs = inputs.draw_problems(39, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        if p.M == 0 or p.N == 0:
            continue
        if p.K == 0:
            assert np.all(got == 0)
            continue
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "few-tiles group %d" % i)


def test_group_single_group_matches_gemm(lib):
    (p,) = inputs.draw_problems(32, [(192, 320, 768)])
    (g1,) = run_group(lib, [p])
    assert np.array_equal(g1, run_gemm(lib, p))


def test_group_many_groups_multiple_launches(lib):
    rng = np.random.default_rng(33)
    shapes = [(int(rng.integers(1, 140)), int(rng.integers(1, 140)), 32 * int(rng.integers(1, 9)))
              for _ in range(150)]
    probs = inputs.draw_problems(34, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "many-group %d" % i)


@pytest.mark.parametrize("route", ["64-row", "128x128"])
def test_group_at_max_groups(lib, route):
    """NVFP4_MAX_GROUPS groups in one call (64 launches), ragged and empty
    groups included, on each side of the planner's M threshold; compared in
    full."""
    rng = np.random.default_rng(41 if route == "64-row" else 45)
    if route == "64-row":
        shapes = [(int(rng.integers(1, 65)), int(rng.integers(1, 100)), 32 * int(rng.integers(0, 13)))
                  for _ in range(lib.NVFP4_MAX_GROUPS)]
        shapes[5], shapes[77] = (0, 64, 256), (17, 0, 64)
    else:
        shapes = [(int(rng.integers(1, 200)), int(rng.integers(1, 200)), 128 * int(rng.integers(1, 4)))
                  for _ in range(lib.NVFP4_MAX_GROUPS)]
        shapes[3], shapes[9] = (200, 130, 256), (0, 64, 128)
    info, _ = lib.group_gemm_plan(shapes)
    assert info["tile_m"] == (64 if route == "64-row" else 128) and info["split_k"] == 1
    probs = inputs.draw_problems(42, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        if p.M == 0 or p.N == 0:
            continue
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "max-groups %s group %d" % (route, i))


@pytest.mark.parametrize("kernel_tile_n,max_n", [(64, 65), (32, 33)])
def test_group_split_k_across_launches(lib, kernel_tile_n, max_n):
    """A K-split plan over more groups than one launch takes: the launches of
    one call share the tile counters and partial tiles, one after the other
    (the 64 x 64 panel and the 64 x 32 stream kernels)."""
    rng = np.random.default_rng(43)
    count = 100 if kernel_tile_n == 64 else 90
    shapes = [(int(rng.integers(1, 65)), int(rng.integers(max_n // 2 + 1, max_n)), 32 * int(rng.integers(128, 193)))
              for _ in range(count)]
    info, _ = lib.group_gemm_plan(shapes)
    assert info["tile_n"] == kernel_tile_n and info["split_k"] > 1
    probs = inputs.draw_problems(44, shapes)
    for rep in range(2):  # the second call finds the counters the first left
        outs = run_group(lib, probs)
        for i, (p, got) in enumerate(zip(probs, outs)):
            c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
            assert_parity(got, c16, bound, "split across launches tile_n %d call %d group %d"
                          % (kernel_tile_n, rep, i))


@pytest.mark.parametrize("index", [3, 4])
def test_full_size_grouped_workloads(lib, index):
    """The 8-group MoE-like and 2-group workloads at full size, as bench.py
    runs them, every output of every group against the oracle."""
    probs = inputs.draw_workload(index)
    outs = run_group(lib, probs)
    for gi, (p, got) in enumerate(zip(probs, outs)):
        check_against_full_oracle(got, p, "%s group %d" % (inputs.WORKLOADS[index].name, gi))


def test_grouped_workload_reduced_full_compare(lib):
    """The 8-group MoE-like shape mix with K cut to 512, compared in full."""
    _, shapes = inputs.workload_shapes(3)
    shapes = [(m, 4096, 512) for (m, _, _) in shapes]
    probs = inputs.draw_problems(35, shapes)
    outs = run_group(lib, probs)
    for gi, (p, got) in enumerate(zip(probs, outs)):
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "moe-reduced group %d" % gi)


# ------------------------------------------------------------ blocked scale layout

@pytest.mark.parametrize("rows,K", [(1, 32), (128, 256), (300, 96), (129, 1056), (512, 7168)])
def test_scales_to_blocked_matches_oracle(lib, rows, K):
    """Every byte of the blocked buffer, padding included, as the oracle's
    layout (the buffer is poisoned first)."""
    rng = np.random.default_rng(rows * 7 + K)
    sf = rng.integers(0, 256, (rows, K // 16), dtype=np.uint8)
    nbytes = lib.nvfp4_blocked_scale_bytes(rows, K)
    blk = torch.full((nbytes,), 0xAB, dtype=torch.uint8, device="cuda")
    lib.nvfp4_scales_to_blocked(to_dev(sf), blk, rows, K)
    torch.cuda.synchronize()
    assert np.array_equal(blk.cpu().numpy(), oracle.scales_to_blocked(sf, rows, K))
    back = torch.full((rows, K // 16), 0xCD, dtype=torch.uint8, device="cuda")
    lib.nvfp4_scales_from_blocked(blk, back, rows, K)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), sf)


def blocked_dev(sf, rows, K):
    return to_dev(oracle.scales_to_blocked(sf, rows, K))


@pytest.mark.parametrize("M,N,K", [
    (64, 6144, 8192),    # panel kernel with a K split (tile counters in the workspace)
    (40, 500, 1024),     # stream kernel (reads the blocked scales directly)
    (300, 260, 2080),    # few tiles with M > 64, ragged K tile: converted scales
])
def test_gemm_blocked_equals_plain(lib, M, N, K):
    p = inputs.draw_problems(5400 + M + K, [(M, N, K)])[0]
    A, SFA, B, SFB, C = dev_problem(p)
    lib.nvfp4_gemm(A, SFA, B, SFB, C, M=M, N=N, K=K)
    torch.cuda.synchronize()
    plain = bits(C)
    C2 = poisoned(M, N)
    lib.nvfp4_gemm_blocked(A, blocked_dev(p.SFA, M, K), B, blocked_dev(p.SFB, N, K), C2, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(bits(C2), plain)
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    assert_parity(plain, c16, bound, "blocked %dx%dx%d" % (M, N, K))


def test_gemm_blocked_direct_equals_plain(lib):
    """306 one-wave 128 x 128 tiles with ragged M and N: the kernel reads the
    blocked scales directly (two atoms per K tile), padding rows included, and
    gives bitwise the plain call's C."""
    M, N, K = 2300, 2170, 1024
    info = lib.gemm_plan(M, N, K)
    assert info["kernel"] == 1 and info["tile_m"] == 128
    p = inputs.draw_problems(5450, [(M, N, K)])[0]
    A, SFA, B, SFB, C = dev_problem(p)
    lib.nvfp4_gemm(A, SFA, B, SFB, C, M=M, N=N, K=K)
    torch.cuda.synchronize()
    plain = bits(C)
    C2 = poisoned(M, N)
    lib.nvfp4_gemm_blocked(A, blocked_dev(p.SFA, M, K), B, blocked_dev(p.SFB, N, K), C2, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(bits(C2), plain)
    check_sampled(plain, p, 5451, "blocked direct %dx%dx%d" % (M, N, K))


def test_group_gemm_blocked_direct(lib):
    """A grouped call on one-wave 128 x 128 tiles (448 tiles, K 256 to 1024,
    an empty group and a K = 0 group) with blocked scales read directly:
    bitwise the plain grouped call, sampled against the oracle."""
    shapes = [(1000, 4096, 512), (300, 4096, 1024), (64, 4096, 256), (0, 64, 256), (130, 4096, 0)]
    info, _ = lib.group_gemm_plan(shapes)
    assert info["kernel"] == 1 and info["tile_m"] == 128
    probs = inputs.draw_problems(43, shapes)
    plain = run_group(lib, probs)
    devs = [dev_problem(p) for p in probs]
    lib.nvfp4_group_gemm_blocked([(d[0], blocked_dev(p.SFA, p.M, p.K) if p.K else d[1], d[2],
                                   blocked_dev(p.SFB, p.N, p.K) if p.K else d[3], d[4], p.M, p.N, p.K)
                                  for d, p in zip(devs, probs)])
    torch.cuda.synchronize()
    for i, (d, p) in enumerate(zip(devs, probs)):
        if p.M == 0 or p.N == 0:
            continue
        got = bits(d[4])
        assert np.array_equal(got, plain[i]), "blocked group %d differs from the plain call" % i
        if p.K == 0:
            assert np.all(got == 0)
            continue
        check_sampled(got, p, 44 + i, "blocked direct group %d" % i)


def test_group_gemm_blocked_then_plain_split(lib):
    """A grouped call with blocked scales, then a plain call that splits K on
    the same stream: the converted scales live past the tile counters, so the
    second call's counters still start at zero."""
    shapes = [(200, 300, 1536), (64, 257, 512), (0, 64, 256), (130, 70, 0)]
    probs = inputs.draw_problems(41, shapes)
    devs = [dev_problem(p) for p in probs]
    lib.nvfp4_group_gemm_blocked([(d[0], blocked_dev(p.SFA, p.M, p.K) if p.K else d[1], d[2],
                                   blocked_dev(p.SFB, p.N, p.K) if p.K else d[3], d[4], p.M, p.N, p.K)
                                  for d, p in zip(devs, probs)])
    torch.cuda.synchronize()
    for i, (d, p) in enumerate(zip(devs, probs)):
        if p.M == 0 or p.N == 0:
            continue
        got = bits(d[4])
        if p.K == 0:
            assert np.all(got == 0)
            continue
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "blocked group %d" % i)
    (q,) = inputs.draw_problems(42, [(64, 64, 16384)])
    assert lib.gemm_plan(64, 64, 16384)["split_k"] > 1
    check_full(lib, q, "split after blocked")


# ------------------------------------------------------------ power-of-two scales
# The FP4-MFMA path for scales that are powers of two: same definition (the
# oracle), inputs restricted to its contract (E4M3 codes with a zero mantissa).

def run_pow2(lib, p):
    A, SFA, B, SFB, C = dev_problem(p)
    lib.nvfp4_gemm_pow2scale(A, SFA, B, SFB, C, M=p.M, N=p.N, K=p.K)
    torch.cuda.synchronize()
    return bits(C)


@pytest.mark.parametrize("M,N,K", [
    (128, 128, 256), (129, 257, 384), (1, 1, 128), (64, 7168, 2048), (300, 520, 1024),
    (256, 384, 4096), (200, 136, 0),
])
def test_pow2scale_matches_oracle(lib, M, N, K):
    p = inputs.draw_problems(5600 + M + K, [(M, N, K)], inputs.POW2_SCALE_CODES)[0]
    got = run_pow2(lib, p)
    if K == 0:
        assert np.all(got == 0)
        return
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    assert_parity(got, c16, bound, "pow2 %dx%dx%d" % (M, N, K))


def test_pow2scale_every_exponent(lib):
    """All fifteen normal power-of-two codes (2^-6 .. 2^8) on each side."""
    codes = np.arange(0x08, 0x79, 8, dtype=np.uint8)
    for side in range(2):
        p = inputs.draw_problems(5700 + side, [(160, 96, 512)], codes)[0]
        # keep the other side small so no sum leaves the fp16 range
        if side == 0:
            p.SFB[:] = 0x08
        else:
            p.SFA[:] = 0x08
        got = run_pow2(lib, p)
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "pow2 exponents side %d" % side)


def test_pow2scale_all_ones_closed_form(lib):
    """Codes 1.0 everywhere give C = K; SFA = 2 gives 2K; SFA = 2^8 with
    SFB = 2^-6 gives 4K (exact in fp16 for these K)."""
    for K, sfa, sfb, scale in [(1024, 0x38, 0x38, 1), (1024, 0x40, 0x38, 2), (512, 0x78, 0x08, 4)]:
        M, N = 130, 70
        A = np.full((M, K // 2), 0x22, np.uint8)
        B = np.full((N, K // 2), 0x22, np.uint8)
        p = inputs.Problem(M, N, K, A, np.full((M, K // 16), sfa, np.uint8), B, np.full((N, K // 16), sfb, np.uint8))
        got = run_pow2(lib, p).view(np.float16).astype(np.float64)
        assert np.all(got == scale * K), (K, sfa, sfb)


def test_group_pow2scale(lib):
    shapes = [(300, 400, 1024), (0, 64, 256), (129, 257, 2048), (200, 100, 0), (64, 640, 512)]
    probs = inputs.draw_problems(5800, shapes, inputs.POW2_SCALE_CODES)
    devs = [dev_problem(p) for p in probs]
    lib.nvfp4_group_gemm_pow2scale([d + (p.M, p.N, p.K) for d, p in zip(devs, probs)])
    torch.cuda.synchronize()
    for i, (d, p) in enumerate(zip(devs, probs)):
        if p.M == 0 or p.N == 0:
            continue
        got = bits(d[4])
        if p.K == 0:
            assert np.all(got == 0)
            continue
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "pow2 group %d" % i)


# ------------------------------------------------------------ batch l and device-resident tables

def test_gemm_batched_matches_oracle(lib):
    """Three batches in dense stacks (the pages' (m, k, l) layout with l
    outermost) against the oracle batch by batch."""
    M, N, K, L = 100, 200, 512, 3
    probs = inputs.draw_problems(5900, [(M, N, K)] * L)
    A = to_dev(np.stack([p.A for p in probs]))
    SFA = to_dev(np.stack([p.SFA for p in probs]))
    B = to_dev(np.stack([p.B for p in probs]))
    SFB = to_dev(np.stack([p.SFB for p in probs]))
    C = torch.full((L, M, N), -1, dtype=torch.int16, device="cuda")
    lib.nvfp4_gemm_batched(A, SFA, B, SFB, C, M, N, K, L)
    torch.cuda.synchronize()
    for i, p in enumerate(probs):
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
        assert_parity(bits(C[i]), c16, bound, "batch %d" % i)


def device_table(lib, rows):
    raw = lib.problem_table_bytes(rows)
    return torch.frombuffer(bytearray(raw), dtype=torch.uint8).cuda()


def tiles_of(shapes):
    return sum(-(-M // 128) * -(-N // 128) for (M, N, K) in shapes if M > 0 and N > 0)


def test_group_gemm_device_table(lib):
    shapes = [(300, 400, 1024), (0, 64, 256), (129, 257, 2048), (200, 100, 0), (64, 640, 512), (1, 1, 128)]
    probs = inputs.draw_problems(5950, shapes)
    devs = [dev_problem(p) for p in probs]
    table = device_table(lib, [d + (p.M, p.N, p.K) for d, p in zip(devs, probs)])
    G = len(shapes)
    ws = torch.empty(lib.nvfp4_group_gemm_device_workspace_bytes(G), dtype=torch.uint8, device="cuda")
    lib.nvfp4_group_gemm_device(table, G, tiles_of(shapes) + 7, ws)
    torch.cuda.synchronize()
    assert list(ws[:16].cpu().numpy().view(np.int32)) == [G, tiles_of(shapes), 0, 0]
    for i, (d, p) in enumerate(zip(devs, probs)):
        if p.M == 0 or p.N == 0:
            continue
        got = bits(d[4])
        if p.K == 0:
            assert np.all(got == 0)
            continue
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "device table group %d" % i)


def test_group_gemm_device_table_skips_entries_outside_contract(lib):
    shapes = [(128, 128, 256), (128, 128, 96), (64, 64, 256)]  # K = 96: not a multiple of 128
    probs = inputs.draw_problems(5960, shapes)
    devs = [dev_problem(p) for p in probs]
    table = device_table(lib, [d + (p.M, p.N, p.K) for d, p in zip(devs, probs)])
    ws = torch.empty(lib.nvfp4_group_gemm_device_workspace_bytes(3), dtype=torch.uint8, device="cuda")
    lib.nvfp4_group_gemm_device(table, 3, 8, ws)
    torch.cuda.synchronize()
    assert list(ws[:16].cpu().numpy().view(np.int32)) == [3, 2, 1, 0]
    assert np.all(bits(devs[1][4]) == 0xFFFF)  # not written
    for i in (0, 2):
        p = probs[i]
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(bits(devs[i][4]), c16, bound, "device table group %d" % i)


def test_group_gemm_device_table_in_graph(lib):
    """Captured once, replayed three times with the groups' M rewritten on the
    device between replays (the table is read at run time); every replay is
    checked against the oracle on the rows it covers."""
    Mmax, N, K, G = 256, 384, 512, 3
    probs = inputs.draw_problems(5970, [(Mmax, N, K)] * G)
    devs = [dev_problem(p) for p in probs]
    table = device_table(lib, [d + (Mmax, N, K) for d in devs])
    words = table.view(torch.int32)  # 14 int32 per 56-byte entry, M at word 10
    ws = torch.empty(lib.nvfp4_group_gemm_device_workspace_bytes(G), dtype=torch.uint8, device="cuda")
    max_tiles = tiles_of([(Mmax, N, K)] * G)
    lib.nvfp4_group_gemm_device(table, G, max_tiles, ws)  # eager run first
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        lib.nvfp4_group_gemm_device(table, G, max_tiles, ws)
    for ms in [(256, 64, 130), (1, 256, 0), (200, 200, 200)]:
        for g_, m in enumerate(ms):
            words[14 * g_ + 10] = m
            devs[g_][4].fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert list(ws[:16].cpu().numpy().view(np.int32)) == [G, tiles_of([(m, N, K) for m in ms]), 0, 0]
        for g_, (m, d, p) in enumerate(zip(ms, devs, probs)):
            got = bits(d[4])
            assert np.all(got[m:] == 0xFFFF), "rows past M written"
            if m == 0:
                continue
            c16, _, bound = oracle.gemm(p.A[:m], p.SFA[:m], p.B, p.SFB, m, N, K)
            assert_parity(got[:m], c16, bound, "graph replay M=%s group %d" % (ms, g_))


@pytest.mark.parametrize("M,N,K,tile_n,split", [
    (64, 1024, 8192, 32, 8),    # stream tile, eight slices (ticket protocol)
    (100, 3072, 4096, 64, 2),   # panel tile, two slices (pair slots)
])
def test_k_split_gemm_under_stream_capture(lib, M, N, K, tile_n, split):
    """A K-split call needs its stream's workspace.  Captured on a stream that
    has none yet it is refused (NOT_SUPPORTED, nothing enqueued); after one
    eager call on that stream the same call captures, and every replay of the
    graph (eager work and synchronisations between them) matches the oracle,
    so each replay leaves the counters and pair slots as it found them."""
    info = lib.gemm_plan(M, N, K)
    assert (info["tile_n"], info["split_k"]) == (tile_n, split) and info["workspace_bytes"] > 0
    p = inputs.draw_problems(6100 + split, [(M, N, K)])[0]
    A, SFA, B, SFB, C = dev_problem(p)
    torch.cuda.synchronize()
    assert lib.release_workspaces() is None  # no stream has a workspace now
    s = torch.cuda.Stream()
    args = (A.data_ptr(), SFA.data_ptr(), B.data_ptr(), SFB.data_ptr(), C.data_ptr(), M, N, K)
    from grouped_gemm_nvfp4_amd import _binding as b
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        rc = b.raw_gemm(*args, s.cuda_stream)
    assert rc == b.NVFP4_ERROR_NOT_SUPPORTED
    torch.cuda.synchronize()
    assert np.all(bits(C) == 0xFFFF), "a refused call enqueued nothing"
    del graph

    with torch.cuda.stream(s):
        assert b.raw_gemm(*args, s.cuda_stream) == b.NVFP4_OK  # allocates the workspace
    torch.cuda.synchronize()
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    assert_parity(bits(C), c16, bound, "eager K-split call")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        rc = b.raw_gemm(*args, s.cuda_stream)
    assert rc == b.NVFP4_OK
    for rep in range(3):
        C.fill_(-1)
        x = torch.ones(1 << 20, device="cuda")  # unrelated eager work between replays
        x.mul_(2.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert_parity(bits(C), c16, bound, "K-split graph replay %d" % rep)


@pytest.mark.parametrize("M,N,K", [
    (4100, 2000, 256),   # ragged M and N, the shortest K (one pair of K tiles), 264 tiles
    (2100, 4000, 512),   # 272 tiles: 256 whole, 16 split in two
    (2537, 4100, 1280),  # odd number of K-tile pairs, 340 tiles, 84 split in three
    (4096, 2048, 2048),  # 256 whole tiles
    (2600, 2600, 1792),  # 231 wide tiles: the 128 x 128 route instead (few tiles)
    (2304, 4096, 1024),  # 288 tiles: 256 whole, 32 split in four
    (2200, 4096, 7168),  # 288 tiles, 32 split in four uneven slices (7, 7, 7, 7 of 28 pairs)
])
def test_wide_tile_shapes(lib, M, N, K):
    """The 128 x 256 wide tile (four waves exchanging decoded A through LDS),
    compared in full, with ragged edges, short and odd K-tile-pair counts, and
    the balancing K split (partial tiles added by the last slice)."""
    info = lib.gemm_plan(M, N, K)
    wide = ((M + 127) // 128) * ((N + 255) // 256) >= 256
    assert info["kernel"] == 4 if wide else info["kernel"] in (1, 3)
    p = inputs.draw_problems(6200 + M + K, [(M, N, K)])[0]
    check_full(lib, p, "wide %dx%dx%d" % (M, N, K))
    assert np.array_equal(run_gemm(lib, p), run_gemm(lib, p)), "wide tile must be deterministic"


def test_wide_tile_group_with_empty_and_zero_k(lib):
    """A grouped wide launch: ragged groups, an empty group, a K = 0 group
    (C is +0) and groups of different K."""
    shapes = [(1700, 2300, 768), (0, 512, 256), (300, 2000, 0), (1025, 777, 256), (129, 3000, 1536),
              (2000, 2570, 512)]
    info, _ = lib.group_gemm_plan(shapes)
    assert info["kernel"] == 4
    probs = inputs.draw_problems(6300, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        if p.M == 0 or p.N == 0:
            continue
        if p.K == 0:
            assert np.all(got == 0), "K = 0 group %d" % i
            continue
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "wide group %d" % i)


def test_group_small_m_wide_tile(lib):
    """A grouped launch on the 64 x 128 small-M tile: ragged groups, a K = 0
    group (zero C), an empty group, different K, and groups of at most 32
    rows (M-edge tiles whose second row block is skipped)."""
    shapes = [(64, 8192, 2048), (40, 8192, 4096), (50, 8000, 1024), (64, 300, 0), (0, 128, 256),
              (64, 320, 2048), (17, 4096, 2048), (32, 1000, 1024)]
    info, _ = lib.group_gemm_plan(shapes)
    assert info["kernel"] == 5 and info["split_k"] == 1
    probs = inputs.draw_problems(40, shapes)
    outs = run_group(lib, probs)
    for i, (p, got) in enumerate(zip(probs, outs)):
        if p.M == 0 or p.N == 0:
            continue
        if p.K == 0:
            assert np.all(got == 0)
            continue
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "small-M wide group %d" % i)


@pytest.mark.parametrize("M,N,K,kernel", [
    (2537, 4100, 1280, 4),   # 128 x 256 tiles, ragged, the tail tiles' K split in three
    (2200, 4096, 7168, 4),   # 288 tiles, 32 split in four; M-edge tiles of one row block
    (33, 30000, 1280, 5),    # 64 x 128 small-M tiles, ragged M and N
    (64, 28672, 4096, 5),
])
def test_shared_decode_tiles_read_blocked_scales(lib, M, N, K, kernel):
    """The shared-decode tiles read blocked scales directly (each wave its
    rows' dwords of the 512-byte atoms, padding rows included): bitwise the
    plain call's C, and within the oracle's tolerance."""
    info = lib.gemm_plan(M, N, K)
    assert info["kernel"] == kernel
    p = inputs.draw_problems(6500 + M + K, [(M, N, K)])[0]
    A, SFA, B, SFB, C = dev_problem(p)
    lib.nvfp4_gemm(A, SFA, B, SFB, C, M=M, N=N, K=K)
    torch.cuda.synchronize()
    plain = bits(C)
    C2 = poisoned(M, N)
    lib.nvfp4_gemm_blocked(A, blocked_dev(p.SFA, M, K), B, blocked_dev(p.SFB, N, K), C2, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(bits(C2), plain), "blocked scales change C"
    if M * N <= 4_000_000:
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
        assert_parity(plain, c16, bound, "blocked shared-decode %dx%dx%d" % (M, N, K))
    else:
        check_sampled(plain, p, 6501 + K, "blocked shared-decode %dx%dx%d" % (M, N, K), plan_tile(lib, M, N, K))


@pytest.mark.parametrize("index", [2, 3, 4])
def test_named_workloads_with_blocked_scales(lib, index):
    """The 8192^3, 8-group MoE and 2-group workloads with blocked scales:
    bitwise the plain calls (every output compared)."""
    probs = inputs.draw_workload(index)
    devs = [dev_problem(p) for p in probs]
    if len(probs) == 1:
        p, d = probs[0], devs[0]
        lib.nvfp4_gemm(*d, M=p.M, N=p.N, K=p.K)
        torch.cuda.synchronize()
        plain = [bits(d[4])]
        C2 = poisoned(p.M, p.N)
        lib.nvfp4_gemm_blocked(d[0], blocked_dev(p.SFA, p.M, p.K), d[2], blocked_dev(p.SFB, p.N, p.K), C2,
                               p.M, p.N, p.K)
        torch.cuda.synchronize()
        got = [bits(C2)]
    else:
        plain = run_group(lib, probs)
        outs = [poisoned(p.M, p.N) for p in probs]
        lib.nvfp4_group_gemm_blocked([(d[0], blocked_dev(p.SFA, p.M, p.K), d[2], blocked_dev(p.SFB, p.N, p.K), o,
                                       p.M, p.N, p.K) for d, p, o in zip(devs, probs, outs)])
        torch.cuda.synchronize()
        got = [bits(o) for o in outs]
    for i, (g_, pl) in enumerate(zip(got, plain)):
        assert np.array_equal(g_, pl), "%s group %d: blocked differs from plain" % (inputs.WORKLOADS[index].name, i)


@pytest.mark.parametrize("M,N,K", [
    (64, 7168, 16384),   # the small-M decode-shaped product, K split in two
    (24, 7168, 8192),    # M <= 32: the one-block form reads only the first dword of each piece
    (300, 512, 16384),   # five row tiles: both halves of the 128-row atoms, padding rows
    (63, 7000, 4608),    # ragged N: the last tile's columns past N
])
def test_panel_reads_blocked_scales(lib, M, N, K):
    """The small-M panel kernel reads blocked scales directly (8-byte halves
    of the atoms' 16-byte lines): bitwise the plain call, and within the
    oracle's tolerance."""
    info = lib.gemm_plan(M, N, K)
    assert info["kernel"] in (1, 2) and (info["tile_m"], info["tile_n"]) == (64, 64)
    p = inputs.draw_problems(6600 + M + K, [(M, N, K)])[0]
    A, SFA, B, SFB, C = dev_problem(p)
    lib.nvfp4_gemm(A, SFA, B, SFB, C, M=M, N=N, K=K)
    torch.cuda.synchronize()
    plain = bits(C)
    C2 = poisoned(M, N)
    lib.nvfp4_gemm_blocked(A, blocked_dev(p.SFA, M, K), B, blocked_dev(p.SFB, N, K), C2, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(bits(C2), plain), "blocked scales change C"
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    assert_parity(plain, c16, bound, "blocked panel %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("M,N,K", [
    (64, 2048, 2048),    # 64 x 32 tiles, K split in two
    (200, 640, 4096),    # four row tiles: both halves of the first atom band, and the second band
    (17, 3000, 1024),    # ragged N: the last tile's columns past N; a quarter of an atom per B tile
])
def test_stream_reads_blocked_scales(lib, M, N, K):
    """The 64 x 32 stream tiles read blocked scales directly (one dword of
    each of a K tile's four atoms per row): bitwise the plain call, and within
    the oracle's tolerance."""
    info = lib.gemm_plan(M, N, K)
    assert (info["tile_m"], info["tile_n"]) == (64, 32)
    p = inputs.draw_problems(6700 + M + K, [(M, N, K)])[0]
    A, SFA, B, SFB, C = dev_problem(p)
    lib.nvfp4_gemm(A, SFA, B, SFB, C, M=M, N=N, K=K)
    torch.cuda.synchronize()
    plain = bits(C)
    C2 = poisoned(M, N)
    lib.nvfp4_gemm_blocked(A, blocked_dev(p.SFA, M, K), B, blocked_dev(p.SFB, N, K), C2, M, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(bits(C2), plain), "blocked scales change C"
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, M, N, K)
    assert_parity(plain, c16, bound, "blocked stream %dx%dx%d" % (M, N, K))


def test_group_panel_reads_blocked_scales(lib):
    """A grouped panel launch with blocked scales (K 256 to 8192, an empty
    group and a K = 0 group): bitwise the plain grouped call."""
    shapes = [(64, 6144, 8192), (40, 4096, 4096), (0, 64, 512), (50, 300, 0), (17, 2304, 256)]
    info, _ = lib.group_gemm_plan(shapes)
    assert (info["tile_m"], info["tile_n"]) == (64, 64)
    probs = inputs.draw_problems(6650, shapes)
    plain = run_group(lib, probs)
    devs = [dev_problem(p) for p in probs]
    outs = [poisoned(p.M, p.N) for p in probs]
    lib.nvfp4_group_gemm_blocked([(d[0], blocked_dev(p.SFA, p.M, p.K) if p.K else d[1], d[2],
                                   blocked_dev(p.SFB, p.N, p.K) if p.K else d[3], o, p.M, p.N, p.K)
                                  for d, p, o in zip(devs, probs, outs)])
    torch.cuda.synchronize()
    for i, (o, p) in enumerate(zip(outs, probs)):
        if p.M == 0 or p.N == 0:
            continue
        got = bits(o)
        assert np.array_equal(got, plain[i]), "blocked group %d differs from the plain call" % i
        if p.K:
            c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
            assert_parity(got, c16, bound, "blocked panel group %d" % i)
