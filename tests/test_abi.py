"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/nvfp4.h declares, rejects bad arguments before touching HIP,
and plans tiles (per-group counts and their exclusive prefix) as documented.
No call here launches work."""
import ctypes
import os
import re

import numpy as np

import pytest

import grouped_gemm_nvfp4_amd as g
from grouped_gemm_nvfp4_amd import _binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_are_exported():
    lib = g.load()
    names = declared_functions()
    assert "nvfp4_gemm" in names and "nvfp4_group_gemm" in names
    for n in names:
        assert hasattr(lib, n), "library does not export %s" % n
    assert sorted(b.EXPORTED) == names


def test_abi_version():
    assert g.abi_version() == 1


def test_binding_constants_match_header():
    text = open(HEADER).read()
    defines = dict(re.findall(r"#define (NVFP4_[A-Z_]+) (-?\d+)", text))
    assert int(defines["NVFP4_MAX_GROUPS"]) == g.NVFP4_MAX_GROUPS
    assert int(defines["NVFP4_MAX_K"]) == g.NVFP4_MAX_K
    assert int(defines["NVFP4_ABI_VERSION"]) == g.abi_version()
    for name in ("NVFP4_OK", "NVFP4_ERROR_INVALID_VALUE", "NVFP4_ERROR_NOT_SUPPORTED", "NVFP4_ERROR_LAUNCH"):
        m = re.search(name + r"\s*=\s*(\d+)", text)
        assert m and int(m.group(1)) == getattr(b, name), name


def test_status_strings():
    for s in range(4):
        assert g.status_string(s).startswith("NVFP4_")
    assert "unknown" in g.status_string(99)


ALIGNED = 1 << 20  # stand-in device address: never dereferenced by these calls


@pytest.mark.parametrize("M,N,K,expect", [
    (-1, 4, 32, b.NVFP4_ERROR_INVALID_VALUE),
    (4, -1, 32, b.NVFP4_ERROR_INVALID_VALUE),
    (4, 4, -32, b.NVFP4_ERROR_INVALID_VALUE),
    (4, 4, 48, b.NVFP4_ERROR_NOT_SUPPORTED),
    (4, 4, 16, b.NVFP4_ERROR_NOT_SUPPORTED),
    (4, 4, b.NVFP4_MAX_K + 32, b.NVFP4_ERROR_NOT_SUPPORTED),
    (4, 4, (1 << 24) + 32, b.NVFP4_ERROR_NOT_SUPPORTED),
    (1 << 30, 1 << 30, 32, b.NVFP4_ERROR_NOT_SUPPORTED),
])
def test_gemm_rejects_bad_sizes(M, N, K, expect):
    assert b.raw_gemm(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, M, N, K, None) == expect


@pytest.mark.parametrize("which", range(5))
def test_gemm_rejects_null_pointers(which):
    ptrs = [ALIGNED] * 5
    ptrs[which] = None
    assert b.raw_gemm(*ptrs, 8, 8, 64, None) == b.NVFP4_ERROR_INVALID_VALUE


def test_gemm_rejects_misaligned_packed_operands():
    assert b.raw_gemm(ALIGNED + 8, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8, 8, 64, None) == \
        b.NVFP4_ERROR_NOT_SUPPORTED
    assert b.raw_gemm(ALIGNED, ALIGNED, ALIGNED + 4, ALIGNED, ALIGNED, 8, 8, 64, None) == \
        b.NVFP4_ERROR_NOT_SUPPORTED


def test_empty_outputs_need_no_pointers():
    # M == 0 or N == 0: a no-op that launches nothing, whatever the pointers
    assert b.raw_gemm(None, None, None, None, None, 0, 5, 64, None) == b.NVFP4_OK
    assert b.raw_gemm(None, None, None, None, None, 5, 0, 64, None) == b.NVFP4_OK


def test_group_rejects_bad_group_counts():
    assert b.raw_group_gemm(None, -1, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert b.raw_group_gemm(None, 3, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert b.raw_group_gemm(None, 0, None) == b.NVFP4_OK
    arr = (b.Nvfp4Problem * 4097)()
    assert b.raw_group_gemm(arr, 4097, None) == b.NVFP4_ERROR_INVALID_VALUE


def test_group_bad_group_fails_whole_call():
    arr = (b.Nvfp4Problem * 3)()
    arr[0] = b.Nvfp4Problem(0, 0, 0, 0, 0, 0, 0, 32)      # empty: fine
    arr[1] = b.Nvfp4Problem(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8, 8, 64)
    arr[2] = b.Nvfp4Problem(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8, 8, 40)
    assert b.raw_group_gemm(arr, 3, None) == b.NVFP4_ERROR_NOT_SUPPORTED
    arr[2] = b.Nvfp4Problem(ALIGNED, None, ALIGNED, ALIGNED, ALIGNED, 8, 8, 64)
    assert b.raw_group_gemm(arr, 3, None) == b.NVFP4_ERROR_INVALID_VALUE


def ceil_div(a, d):
    return -(-a // d)


def test_plan_single():
    info = g.gemm_plan(8192, 8192, 8192)
    assert info["kernel"] == 4 and (info["tile_m"], info["tile_n"]) == (128, 256)
    tm, tn = info["tile_m"], info["tile_n"]
    assert info["total_tiles"] == ceil_div(8192, tm) * ceil_div(8192, tn)
    assert info["workgroups"] == info["total_tiles"] * info["split_k"]
    assert g.gemm_plan(0, 10, 64)["kernel"] == 0


def test_plan_group_prefix_is_exclusive_scan_of_tile_counts():
    shapes = [(64, 4096, 7168), (0, 4096, 7168), (512, 4096, 7168), (1, 1, 32),
              (384, 3072, 1536), (5, 0, 32)]
    info, prefix = g.group_gemm_plan(shapes)
    tm, tn = info["tile_m"], info["tile_n"]
    counts = [0 if (M == 0 or N == 0) else ceil_div(M, tm) * ceil_div(N, tn)
              for (M, N, _) in shapes]
    expect = [0]
    for c in counts:
        expect.append(expect[-1] + c)
    assert prefix == expect
    assert info["total_tiles"] == expect[-1]


@pytest.mark.parametrize("M,N,K,tile_m", [
    (64, 7168, 16384, 64),     # M <= 64: 64-row kernels
    (128, 128, 256, 64),       # one 128 x 128 tile: 64-row kernels
    (2048, 1024, 4096, 64),    # 128 tiles of 128 x 128: still the 64-row kernels
    (2048, 1152, 4096, 128),   # 144 tiles: 128 x 128 tiles
    (8192, 8192, 8192, 128),   # 4096 tiles
])
def test_plan_tile_rows_follow_the_128_tile_count(M, N, K, tile_m):
    """Launches with M > 64 and at most 128 tiles of 128 x 128 take the 64-row
    kernels; larger ones take 128-row tiles (128 x 256 wide tiles when every
    K % 256 == 0, else 128 x 128)."""
    assert g.gemm_plan(M, N, K)["tile_m"] == tile_m


def test_plan_group_tile_rows_count_all_groups():
    """The 128-tile limit is on the whole launch: 4 groups of 32 tiles fit
    under it, 5 do not."""
    assert g.group_gemm_plan([(128, 4096, 1024)] * 4)[0]["tile_m"] == 64
    assert g.group_gemm_plan([(128, 4096, 1024)] * 5)[0]["tile_m"] == 128


def test_plan_errors_match_call_errors():
    with pytest.raises(g.Nvfp4Error) as e:
        g.gemm_plan(4, 4, 48)
    assert e.value.status == b.NVFP4_ERROR_NOT_SUPPORTED
    with pytest.raises(g.Nvfp4Error):
        g.group_gemm_plan([(4, 4, 32), (-1, 4, 32)])


def test_problem_struct_matches_header_layout():
    # 5 pointers then 3 ints, natural alignment
    assert ctypes.sizeof(b.Nvfp4Problem) == 5 * 8 + 3 * 4 + 4
    assert b.Nvfp4Problem.M.offset == 40


# ------------------------------------------------------------ blocked scale layout

@pytest.mark.parametrize("rows,K", [(0, 64), (1, 32), (128, 256), (129, 96), (300, 7168), (5, 0)])
def test_blocked_scale_bytes_match_the_layout(rows, K):
    import oracle
    assert b.nvfp4_blocked_scale_bytes(rows, K) == oracle.blocked_scale_shape(rows, K)[2]


@pytest.mark.parametrize("rows,K", [(-1, 32), (4, -32), (4, 48), (4, (1 << 24) + 32)])
def test_blocked_scale_bytes_reject_bad_sizes(rows, K):
    assert b.nvfp4_blocked_scale_bytes(rows, K) == -1


@pytest.mark.parametrize("fn", ["nvfp4_scales_to_blocked", "nvfp4_scales_from_blocked"])
def test_scale_conversion_rejects_bad_arguments(fn):
    f = getattr(g.load(), fn)
    assert f(ALIGNED, ALIGNED, -1, 64, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, ALIGNED, 4, 48, None) == b.NVFP4_ERROR_NOT_SUPPORTED
    assert f(None, ALIGNED, 4, 64, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, None, 4, 64, None) == b.NVFP4_ERROR_INVALID_VALUE
    # the blocked side moves in 16-byte pieces: it must be 16-byte aligned
    for off in (2, 4, 8):
        if fn == "nvfp4_scales_to_blocked":
            assert f(ALIGNED, ALIGNED + off, 4, 64, None) == b.NVFP4_ERROR_INVALID_VALUE
        else:
            assert f(ALIGNED + off, ALIGNED, 4, 64, None) == b.NVFP4_ERROR_INVALID_VALUE
    # nothing to move: no launch, no pointer needed
    assert f(None, None, 0, 64, None) == b.NVFP4_OK
    assert f(None, None, 7, 0, None) == b.NVFP4_OK


def test_blocked_gemm_rejects_bad_arguments():
    lib = g.load()
    assert lib.nvfp4_gemm_blocked(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8, 8, 48, None) == \
        b.NVFP4_ERROR_NOT_SUPPORTED
    assert lib.nvfp4_gemm_blocked(ALIGNED, None, ALIGNED, ALIGNED, ALIGNED, 8, 8, 64, None) == \
        b.NVFP4_ERROR_INVALID_VALUE
    assert lib.nvfp4_gemm_blocked(ALIGNED, ALIGNED + 1, ALIGNED, ALIGNED, ALIGNED, 8, 8, 64, None) == \
        b.NVFP4_ERROR_INVALID_VALUE
    assert lib.nvfp4_gemm_blocked(ALIGNED, ALIGNED, ALIGNED, ALIGNED + 8, ALIGNED, 8, 8, 64, None) == \
        b.NVFP4_ERROR_INVALID_VALUE
    assert lib.nvfp4_gemm_blocked(None, None, None, None, None, 0, 8, 64, None) == b.NVFP4_OK
    assert lib.nvfp4_group_gemm_blocked(None, 0, None) == b.NVFP4_OK


# ------------------------------------------------------------ power-of-two scales
def test_pow2scale_gemm_rejects_bad_arguments():
    """Argument errors come back before any HIP call (no GPU needed)."""
    lib = g.load()
    # the FP4-MFMA path takes whole 128-K tiles and 8-byte aligned scale rows
    assert lib.nvfp4_gemm_pow2scale(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8, 8, 96, None) == \
        b.NVFP4_ERROR_NOT_SUPPORTED
    assert lib.nvfp4_gemm_pow2scale(ALIGNED, ALIGNED + 4, ALIGNED, ALIGNED, ALIGNED, 8, 8, 128, None) == \
        b.NVFP4_ERROR_NOT_SUPPORTED
    assert lib.nvfp4_gemm_pow2scale(ALIGNED, ALIGNED, ALIGNED, ALIGNED + 2, ALIGNED, 8, 8, 256, None) == \
        b.NVFP4_ERROR_NOT_SUPPORTED
    # the general rules still apply first
    assert lib.nvfp4_gemm_pow2scale(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8, 8, 48, None) == \
        b.NVFP4_ERROR_NOT_SUPPORTED
    assert lib.nvfp4_gemm_pow2scale(ALIGNED, None, ALIGNED, ALIGNED, ALIGNED, 8, 8, 128, None) == \
        b.NVFP4_ERROR_INVALID_VALUE
    assert lib.nvfp4_gemm_pow2scale(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, -1, 8, 128, None) == \
        b.NVFP4_ERROR_INVALID_VALUE
    # nothing to do: no launch
    assert lib.nvfp4_gemm_pow2scale(None, None, None, None, None, 0, 8, 128, None) == b.NVFP4_OK
    assert lib.nvfp4_group_gemm_pow2scale(None, 0, None) == b.NVFP4_OK
    assert lib.nvfp4_group_gemm_pow2scale(None, 1, None) == b.NVFP4_ERROR_INVALID_VALUE


# ------------------------------------------------------------ batch l and device-resident tables
def test_batched_rejects_bad_arguments():
    lib = g.load()
    f = lib.nvfp4_gemm_batched
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8, 8, 64, -1, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, -8, 8, 64, 2, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8, 8, 64, 4097, None) == b.NVFP4_ERROR_NOT_SUPPORTED
    assert f(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 8, 8, 48, 3, None) == b.NVFP4_ERROR_NOT_SUPPORTED
    assert f(ALIGNED, None, ALIGNED, ALIGNED, ALIGNED, 8, 8, 64, 3, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(None, None, None, None, None, 8, 8, 64, 0, None) == b.NVFP4_OK
    assert f(None, None, None, None, None, 0, 8, 64, 5, None) == b.NVFP4_OK


@pytest.mark.parametrize("G", [0, 1, 2, 7, 64, 4096])
def test_device_table_workspace_bytes(G):
    # header (16 bytes), G + 1 prefix ints, rounded up to 16, then one
    # 56-byte problem descriptor (5 pointers, 4 ints) per group
    expect = (16 + 4 * (G + 1) + 15) // 16 * 16 + 56 * G
    assert b.nvfp4_group_gemm_device_workspace_bytes(G) == expect


def test_device_table_workspace_bytes_rejects_bad_counts():
    assert b.nvfp4_group_gemm_device_workspace_bytes(-1) == -1
    assert b.nvfp4_group_gemm_device_workspace_bytes(4097) == -1


def test_device_table_call_rejects_bad_arguments():
    lib = g.load()
    f = lib.nvfp4_group_gemm_device
    need = b.nvfp4_group_gemm_device_workspace_bytes(3)
    assert f(ALIGNED, -1, 10, ALIGNED, need, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, 4097, 10, ALIGNED, 10 ** 9, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, 3, -1, ALIGNED, need, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(None, 3, 10, ALIGNED, need, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, 3, 10, None, need, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, 3, 10, ALIGNED + 8, need, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, 3, 10, ALIGNED, need - 1, None) == b.NVFP4_ERROR_INVALID_VALUE
    assert f(ALIGNED, 3, 1 << 24, ALIGNED, need, None) == b.NVFP4_ERROR_NOT_SUPPORTED
    # nothing to enqueue
    assert f(None, 0, 10, None, 0, None) == b.NVFP4_OK
    assert f(ALIGNED, 3, 0, ALIGNED, need, None) == b.NVFP4_OK


def test_problem_table_bytes_layout():
    raw = b.problem_table_bytes([(16, 32, 48, 64, 80, 1, 2, 128), (None, None, None, None, None, 0, 0, 0)])
    assert len(raw) == 2 * 56
    words = np.frombuffer(raw[:56], dtype=np.uint64)[:5]
    assert list(words) == [16, 32, 48, 64, 80]
    assert list(np.frombuffer(raw[40:52], dtype=np.int32)) == [1, 2, 128]


def test_k_limit_is_the_accuracy_bound():
    """K up to NVFP4_MAX_K plans; one block of 32 more is refused, by the
    plain, blocked and power-of-two entry points alike."""
    K = g.NVFP4_MAX_K
    assert g.gemm_plan(64, 64, K)["workgroups"] > 0
    assert g.gemm_plan(256, 16512, K)["tile_m"] == 128
    for fn in (b.raw_gemm,):
        assert fn(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 4, 4, K + 32, None) == b.NVFP4_ERROR_NOT_SUPPORTED
    lib = g.load()
    for name in ("nvfp4_gemm_blocked", "nvfp4_gemm_pow2scale"):
        fn = getattr(lib, name)
        assert fn(ALIGNED, ALIGNED, ALIGNED, ALIGNED, ALIGNED, 4, 4, K + 128, None) == b.NVFP4_ERROR_NOT_SUPPORTED
    # the worst-case accumulated error bound at the limit, as nvfp4.h states it
    assert K * 2.0 ** -27 + 2.0 ** -19 < 1e-3


@pytest.mark.parametrize("M,N,K,kernel,tile_n", [
    (8192, 8192, 8192, 4, 256),    # K % 256 == 0: the wide 128 x 256 tile
    (2048, 1152, 4224, 3, 128),    # K % 256 != 0: 128 x 128 tiles (here four waves per tile)
    (1024, 65536, 128, 1, 128),    # K % 256 != 0, many tiles: one wave per 128 x 128 tile
])
def test_plan_wide_tile_needs_k_multiple_of_256(M, N, K, kernel, tile_n):
    info = g.gemm_plan(M, N, K)
    assert (info["kernel"], info["tile_m"], info["tile_n"]) == (kernel, 128, tile_n)
    assert info["total_tiles"] == ceil_div(M, 128) * ceil_div(N, tile_n)
    assert info["split_k"] == 1 and info["workspace_bytes"] == 0


@pytest.mark.parametrize("M,N,K,workgroups,split", [
    (8192, 8192, 8192, 2048, 1),   # 2048 tiles: several rounds of whole tiles
    (4096, 3072, 7168, 512, 2),    # 384 tiles: 256 whole, the other 128 split in two
    (2304, 4096, 1024, 384, 4),    # 288 tiles: 256 whole, the other 32 split in four
    (8192, 2048, 256, 512, 1),     # K = 256: one pair of K tiles, nothing to split
])
def test_plan_wide_balance(M, N, K, workgroups, split):
    """Wide launches of fewer than 1024 tiles run whole tiles in rounds of
    one per CU and split the K of the rest over the CUs."""
    info = g.gemm_plan(M, N, K)
    assert info["kernel"] == 4
    assert info["workgroups"] == workgroups and info["split_k"] == split
    slots = workgroups - (info["total_tiles"] // 256 * 256) if split > 1 else 0
    # tile counters (4096 x 4 bytes), the two-slice pair slots (128 tiles of
    # 64 x 64 words), then one 128 x 256 fp32 partial tile per split slot
    assert info["workspace_bytes"] == (16384 + 128 * 64 * 64 * 4 + slots * 128 * 256 * 4 if slots else 0)


def test_plan_grouped_workloads_take_the_wide_tile():
    """The 8-group MoE (304 tiles) and the 2-group workload (384 + 36 tiles):
    one whole tile per CU, the rest split (the 2-group workload's short-K
    group stays whole: its tiles are shorter than the slice length)."""
    from grouped_gemm_nvfp4_amd import inputs
    info, prefix = g.group_gemm_plan(inputs.workload_shapes(3)[1])
    assert info["kernel"] == 4 and info["tile_n"] == 256 and prefix[-1] == info["total_tiles"] == 304
    assert info["split_k"] == 4 and info["workgroups"] == 256 + 48 * 4
    info, prefix = g.group_gemm_plan(inputs.workload_shapes(4)[1])
    assert info["kernel"] == 4 and prefix[-1] == info["total_tiles"] == 420
    assert info["split_k"] == 2 and info["workgroups"] == 256 + 128 * 2 + 36


def test_plan_wide_tile_needs_a_tile_per_cu():
    """Fewer than 256 wide tiles: the 128 x 128 route (here four waves per
    tile), not the wide tile with its K split."""
    info = g.gemm_plan(2048, 2048, 2048)
    assert info["kernel"] == 3 and info["tile_n"] == 128
    assert g.gemm_plan(4096, 2048, 2048)["kernel"] == 4  # 256 wide tiles


def test_two_slice_panel_plans_fit_the_pair_slots():
    """Two-slice launches of the 64 x 64 panel tile sum through the library
    workspace's pair slots, one 32-bit word per output element of at most 128
    tiles (2 MiB between the tile counters and the partial tiles).  Over seeded
    random single and grouped shapes in the 64-row regimes, every such plan
    stays within 128 tiles and asks for the counters, the pair slots and two
    16 KiB partial tiles per tile."""
    rng = np.random.default_rng(77)
    pair_bytes = 128 * 64 * 64 * 4
    seen = 0
    for _ in range(400):
        G = int(rng.integers(1, 4))
        shapes = [(int(rng.integers(1, 400)), int(rng.integers(1, 9000)), 256 * int(rng.integers(1, 64)))
                  for _ in range(G)]
        info, _ = g.group_gemm_plan(shapes)
        if info["kernel"] == 2 and info["tile_n"] == 64 and info["split_k"] == 2:
            seen += 1
            assert info["total_tiles"] <= 128, shapes
            assert info["workspace_bytes"] == 16384 + pair_bytes + info["total_tiles"] * 2 * 64 * 64 * 4
    assert seen >= 10  # the sweep reaches the two-slice panel plans
