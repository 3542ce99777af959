"""The allocation-free entry point nvfp4_gemm_noalloc, through the C ABI.

Its output must equal nvfp4_gemm's (same plan, same kernels) bit for bit and
meet the oracle's parity rule, on consecutive calls that share the per-GPU
scratch array: a K-split call, then a smaller K-split call that finds the
array as the first left it.  It also captures on a fresh stream, where
nvfp4_gemm's K-split calls are refused.
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


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _operands(p):
    return (_dev(p.A), _dev(p.SFA), _dev(p.B), _dev(p.SFB))


def _poisoned(M, N):
    return torch.full((M, N), -1, dtype=torch.int16, device="cuda")  # 0xFFFF


def _bits(C):
    return C.cpu().numpy().view(np.uint16)


def _call(fn, ops, C, p, stream):
    A, SFA, B, SFB = ops
    return fn(A.data_ptr(), SFA.data_ptr(), B.data_ptr(), SFB.data_ptr(), C.data_ptr(), p.M, p.N, p.K, stream)


def test_noalloc_equals_gemm_on_consecutive_calls(lib):
    from grouped_gemm_nvfp4_amd import _binding as b
    shapes = [(64, 7168, 16384), (33, 513, 8192)]  # the second smaller, both split K
    probs = inputs.draw_problems(7100, shapes)
    sh = torch.cuda.current_stream().cuda_stream
    for p in probs:
        info = lib.gemm_plan(p.M, p.N, p.K)
        assert info["split_k"] > 1 and 0 < info["workspace_bytes"] <= 16384 + 8388608
        ops = _operands(p)
        C_ref, C_na = _poisoned(p.M, p.N), _poisoned(p.M, p.N)
        assert _call(b.raw_gemm, ops, C_ref, p, sh) == b.NVFP4_OK
        assert _call(b.raw_gemm_noalloc, ops, C_na, p, sh) == b.NVFP4_OK
        torch.cuda.synchronize()
        ref, got = _bits(C_ref), _bits(C_na)
        assert np.array_equal(got, ref), "noalloc differs from nvfp4_gemm at %s" % ((p.M, p.N, p.K),)
        c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
        assert_parity(got, c16, bound, "noalloc %dx%dx%d" % (p.M, p.N, p.K))


def test_noalloc_without_k_split_and_empty(lib):
    from grouped_gemm_nvfp4_amd import _binding as b
    sh = torch.cuda.current_stream().cuda_stream
    p = inputs.draw_problems(7101, [(300, 520, 1024)])[0]
    info = lib.gemm_plan(p.M, p.N, p.K)
    ops = _operands(p)
    C_ref, C_na = _poisoned(p.M, p.N), _poisoned(p.M, p.N)
    assert _call(b.raw_gemm, ops, C_ref, p, sh) == b.NVFP4_OK
    assert _call(b.raw_gemm_noalloc, ops, C_na, p, sh) == b.NVFP4_OK
    torch.cuda.synchronize()
    assert np.array_equal(_bits(C_na), _bits(C_ref)), "plan %s" % (info,)
    assert b.raw_gemm_noalloc(None, None, None, None, C_na.data_ptr(), 0, 5, 64, sh) == b.NVFP4_OK
    assert b.raw_gemm_noalloc(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 4, 4, 48, sh) == \
        b.NVFP4_ERROR_NOT_SUPPORTED


def test_noalloc_captures_on_a_fresh_stream(lib):
    """No workspace to allocate: the K-split call captures on a stream the
    library has never seen, and every replay matches nvfp4_gemm."""
    from grouped_gemm_nvfp4_amd import _binding as b
    p = inputs.draw_problems(7102, [(64, 1024, 8192)])[0]
    assert lib.gemm_plan(p.M, p.N, p.K)["split_k"] > 1
    ops = _operands(p)
    C_ref, C_na = _poisoned(p.M, p.N), _poisoned(p.M, p.N)
    assert _call(b.raw_gemm, ops, C_ref, p, torch.cuda.current_stream().cuda_stream) == b.NVFP4_OK
    torch.cuda.synchronize()
    lib.release_workspaces()
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        rc = _call(b.raw_gemm_noalloc, ops, C_na, p, s.cuda_stream)
    assert rc == b.NVFP4_OK
    for rep in range(3):
        C_na.fill_(-1)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(_bits(C_na), _bits(C_ref)), "replay %d" % rep


def test_noalloc_keeps_wide_tiles_whole_when_the_split_does_not_fit(lib):
    """4096 x 3072 x 7168 (384 wide tiles): nvfp4_gemm splits the K of the 128
    tiles past one round in two (32 MiB of partial tiles); the allocation-free
    call keeps the tiles whole.  Both meet the oracle's parity rule."""
    from grouped_gemm_nvfp4_amd import _binding as b
    p = inputs.draw_problems(7103, [(4096, 3072, 7168)])[0]
    info = lib.gemm_plan(p.M, p.N, p.K)
    assert info["kernel"] == 4 and info["workspace_bytes"] > 16384 + 8388608
    sh = torch.cuda.current_stream().cuda_stream
    ops = _operands(p)
    C_ref, C_na = _poisoned(p.M, p.N), _poisoned(p.M, p.N)
    assert _call(b.raw_gemm, ops, C_ref, p, sh) == b.NVFP4_OK
    assert _call(b.raw_gemm_noalloc, ops, C_na, p, sh) == b.NVFP4_OK
    torch.cuda.synchronize()
    c16, _, bound = oracle.gemm(p.A, p.SFA, p.B, p.SFB, p.M, p.N, p.K)
    assert_parity(_bits(C_ref), c16, bound, "gemm 4096x3072x7168")
    assert_parity(_bits(C_na), c16, bound, "noalloc 4096x3072x7168")
