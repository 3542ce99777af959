"""ctypes binding of ``libnvfp4.so`` (the C ABI in include/nvfp4.h).

Argument marshalling only: every step of the computation runs in the
library's gfx950 kernels.  Tensors are passed as raw device pointers together
with their sizes and torch's current HIP stream.  A missing library raises
immediately; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libnvfp4.so")

NVFP4_OK = 0
NVFP4_ERROR_INVALID_VALUE = 1
NVFP4_ERROR_NOT_SUPPORTED = 2
NVFP4_ERROR_LAUNCH = 3
NVFP4_MAX_GROUPS = 4096  # groups per grouped call
NVFP4_MAX_K = 131072  # largest K of a product (the accuracy bound)

EXPORTED = [
    "nvfp4_gemm", "nvfp4_group_gemm", "nvfp4_gemm_plan", "nvfp4_group_gemm_plan",
    "nvfp4_release_workspaces", "nvfp4_status_string", "nvfp4_abi_version",
    "nvfp4_blocked_scale_bytes", "nvfp4_scales_to_blocked", "nvfp4_scales_from_blocked",
    "nvfp4_gemm_blocked", "nvfp4_group_gemm_blocked",
    "nvfp4_gemm_pow2scale", "nvfp4_group_gemm_pow2scale",
    "nvfp4_gemm_batched", "nvfp4_group_gemm_device_workspace_bytes", "nvfp4_group_gemm_device",
    "nvfp4_gemm_noalloc",
]


class Nvfp4Problem(ctypes.Structure):
    _fields_ = [("A", ctypes.c_void_p), ("SFA", ctypes.c_void_p),
                ("B", ctypes.c_void_p), ("SFB", ctypes.c_void_p),
                ("C", ctypes.c_void_p), ("M", ctypes.c_int), ("N", ctypes.c_int),
                ("K", ctypes.c_int)]


class Nvfp4PlanInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int), ("tile_m", ctypes.c_int),
                ("tile_n", ctypes.c_int), ("split_k", ctypes.c_int),
                ("total_tiles", ctypes.c_int), ("workgroups", ctypes.c_int),
                ("workspace_bytes", ctypes.c_longlong)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(text)
        self.status = status


_lib = None


def load():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libnvfp4.so is not built (%s); run `python -m grouped_gemm_nvfp4_amd.build`"
            % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.nvfp4_gemm.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp]
    lib.nvfp4_gemm.restype = ci
    lib.nvfp4_group_gemm.argtypes = [ctypes.POINTER(Nvfp4Problem), ci, vp]
    lib.nvfp4_group_gemm.restype = ci
    lib.nvfp4_gemm_plan.argtypes = [ci, ci, ci, ctypes.POINTER(Nvfp4PlanInfo)]
    lib.nvfp4_gemm_plan.restype = ci
    lib.nvfp4_group_gemm_plan.argtypes = [ctypes.POINTER(Nvfp4Problem), ci,
                                          ctypes.POINTER(Nvfp4PlanInfo),
                                          ctypes.POINTER(ctypes.c_int)]
    lib.nvfp4_group_gemm_plan.restype = ci
    lib.nvfp4_release_workspaces.argtypes = []
    lib.nvfp4_release_workspaces.restype = ci
    lib.nvfp4_status_string.argtypes = [ci]
    lib.nvfp4_status_string.restype = ctypes.c_char_p
    lib.nvfp4_abi_version.argtypes = []
    lib.nvfp4_abi_version.restype = ci
    lib.nvfp4_blocked_scale_bytes.argtypes = [ci, ci]
    lib.nvfp4_blocked_scale_bytes.restype = ctypes.c_longlong
    lib.nvfp4_scales_to_blocked.argtypes = [vp, vp, ci, ci, vp]
    lib.nvfp4_scales_to_blocked.restype = ci
    lib.nvfp4_scales_from_blocked.argtypes = [vp, vp, ci, ci, vp]
    lib.nvfp4_scales_from_blocked.restype = ci
    lib.nvfp4_gemm_blocked.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp]
    lib.nvfp4_gemm_blocked.restype = ci
    lib.nvfp4_group_gemm_blocked.argtypes = [ctypes.POINTER(Nvfp4Problem), ci, vp]
    lib.nvfp4_group_gemm_blocked.restype = ci
    lib.nvfp4_gemm_batched.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, vp]
    lib.nvfp4_gemm_batched.restype = ci
    lib.nvfp4_group_gemm_device_workspace_bytes.argtypes = [ci]
    lib.nvfp4_group_gemm_device_workspace_bytes.restype = ctypes.c_longlong
    lib.nvfp4_group_gemm_device.argtypes = [vp, ci, ci, vp, ctypes.c_longlong, vp]
    lib.nvfp4_group_gemm_device.restype = ci
    lib.nvfp4_gemm_pow2scale.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp]
    lib.nvfp4_gemm_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, vp]
    lib.nvfp4_gemm_noalloc.restype = ci
    lib.nvfp4_gemm_pow2scale.restype = ci
    lib.nvfp4_group_gemm_pow2scale.argtypes = [ctypes.POINTER(Nvfp4Problem), ci, vp]
    lib.nvfp4_group_gemm_pow2scale.restype = ci
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().nvfp4_status_string(status).decode()


def _check(status: int):
    if status != NVFP4_OK:
        raise Nvfp4Error(status, status_string(status))


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _problem(A, SFA, B, SFB, C, M, N, K) -> Nvfp4Problem:
    return Nvfp4Problem(_ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB), _ptr(C), M, N, K)


def _sizes(A, B, C):
    M, N = C.shape[0], C.shape[1]
    K = 2 * A.shape[1] if A is not None and A.dim() == 2 else 0
    return int(M), int(N), int(K)


def nvfp4_gemm(A, SFA, B, SFB, C, M=None, N=None, K=None, stream=None):
    """C[M][N] (fp16) = NVFP4 product of A [M][K/2], SFA [M][K/16], B [N][K/2],
    SFB [N][K/16] (uint8 tensors on the GPU).  Asynchronous on ``stream``
    (torch's current stream by default).  Raises Nvfp4Error on a bad status."""
    if M is None:
        M, N, K = _sizes(A, B, C)
    _check(load().nvfp4_gemm(_ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB), _ptr(C),
                             M, N, K, _stream_handle(stream)))


def nvfp4_group_gemm(problems, stream=None):
    """Grouped product in one launch.  ``problems`` is a sequence of
    (A, SFA, B, SFB, C) tensor tuples or (A, SFA, B, SFB, C, M, N, K)."""
    arr = (Nvfp4Problem * max(1, len(problems)))()
    for i, p in enumerate(problems):
        if len(p) == 5:
            A, SFA, B, SFB, C = p
            M, N, K = _sizes(A, B, C)
        else:
            A, SFA, B, SFB, C, M, N, K = p
        arr[i] = _problem(A, SFA, B, SFB, C, M, N, K)
    _check(load().nvfp4_group_gemm(arr, len(problems), _stream_handle(stream)))


def nvfp4_gemm_blocked(A, SFA, B, SFB, C, M, N, K, stream=None):
    """nvfp4_gemm with SFA and SFB in the blocked layout (uint8 device
    tensors of nvfp4_blocked_scale_bytes(M or N, K) bytes)."""
    _check(load().nvfp4_gemm_blocked(_ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB), _ptr(C),
                                     M, N, K, _stream_handle(stream)))


def nvfp4_group_gemm_blocked(problems, stream=None):
    """nvfp4_group_gemm with blocked scales; ``problems`` as for
    nvfp4_group_gemm with explicit (A, SFA, B, SFB, C, M, N, K)."""
    arr = (Nvfp4Problem * max(1, len(problems)))()
    for i, (A, SFA, B, SFB, C, M, N, K) in enumerate(problems):
        arr[i] = _problem(A, SFA, B, SFB, C, M, N, K)
    _check(load().nvfp4_group_gemm_blocked(arr, len(problems), _stream_handle(stream)))


def nvfp4_gemm_pow2scale(A, SFA, B, SFB, C, M, N, K, stream=None):
    """nvfp4_gemm for scales that are all powers of two (E4M3 codes with a
    zero mantissa and a nonzero exponent field), on the scaled FP4 MFMA."""
    _check(load().nvfp4_gemm_pow2scale(_ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB), _ptr(C),
                                       M, N, K, _stream_handle(stream)))


def nvfp4_group_gemm_pow2scale(problems, stream=None):
    """nvfp4_group_gemm for power-of-two scales; ``problems`` as for
    nvfp4_group_gemm with explicit (A, SFA, B, SFB, C, M, N, K)."""
    arr = (Nvfp4Problem * max(1, len(problems)))()
    for i, (A, SFA, B, SFB, C, M, N, K) in enumerate(problems):
        arr[i] = _problem(A, SFA, B, SFB, C, M, N, K)
    _check(load().nvfp4_group_gemm_pow2scale(arr, len(problems), _stream_handle(stream)))


def nvfp4_gemm_batched(A, SFA, B, SFB, C, M, N, K, L, stream=None):
    """L products of the same sizes over dense stacks of operands (batch b of A
    at byte b*M*K/2, and so on)."""
    _check(load().nvfp4_gemm_batched(_ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB), _ptr(C),
                                     M, N, K, L, _stream_handle(stream)))


def problem_table_bytes(problems) -> bytes:
    """The raw bytes of an nvfp4_problem array, for a device-resident table:
    ``problems`` is a sequence of (A, SFA, B, SFB, C, M, N, K) with tensors or
    integer addresses."""
    arr = (Nvfp4Problem * max(1, len(problems)))()
    for i, (A, SFA, B, SFB, C, M, N, K) in enumerate(problems):
        addr = [x if isinstance(x, int) or x is None else x.data_ptr() for x in (A, SFA, B, SFB, C)]
        arr[i] = Nvfp4Problem(*addr, M, N, K)
    return bytes(arr)[:ctypes.sizeof(Nvfp4Problem) * len(problems)]


def nvfp4_group_gemm_device_workspace_bytes(num_groups) -> int:
    return int(load().nvfp4_group_gemm_device_workspace_bytes(num_groups))


def nvfp4_group_gemm_device(table, num_groups, max_tiles, workspace, stream=None):
    """Grouped product whose problem table ``table`` (a device uint8 tensor
    holding num_groups nvfp4_problem entries) is read on the device; the plan
    goes into ``workspace`` (a device tensor of at least
    nvfp4_group_gemm_device_workspace_bytes(num_groups) bytes)."""
    _check(load().nvfp4_group_gemm_device(_ptr(table), num_groups, max_tiles, _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream_handle(stream)))


def nvfp4_blocked_scale_bytes(rows, K) -> int:
    return int(load().nvfp4_blocked_scale_bytes(rows, K))


def nvfp4_scales_to_blocked(sf, blocked, rows, K, stream=None):
    _check(load().nvfp4_scales_to_blocked(_ptr(sf), _ptr(blocked), rows, K, _stream_handle(stream)))


def nvfp4_scales_from_blocked(blocked, sf, rows, K, stream=None):
    _check(load().nvfp4_scales_from_blocked(_ptr(blocked), _ptr(sf), rows, K, _stream_handle(stream)))


def raw_gemm(A, SFA, B, SFB, C, M, N, K, stream) -> int:
    """The C entry point with raw integer pointers; returns the status code."""
    return load().nvfp4_gemm(A, SFA, B, SFB, C, M, N, K, stream)


def raw_gemm_noalloc(A, SFA, B, SFB, C, M, N, K, stream) -> int:
    """nvfp4_gemm_noalloc with raw integer pointers; returns the status code."""
    return load().nvfp4_gemm_noalloc(A, SFA, B, SFB, C, M, N, K, stream)


def nvfp4_gemm_noalloc(A, SFA, B, SFB, C, M=None, N=None, K=None, stream=None):
    """nvfp4_gemm without any device allocation (K-split scratch in the
    library's per-GPU static array); raises Nvfp4Error on a bad status."""
    if M is None:
        M, N, K = _sizes(A, B, C)
    _check(load().nvfp4_gemm_noalloc(_ptr(A), _ptr(SFA), _ptr(B), _ptr(SFB), _ptr(C),
                                     M, N, K, _stream_handle(stream)))


def raw_group_gemm(problems, num_groups, stream) -> int:
    """``problems``: a ctypes array of Nvfp4Problem (or None); returns the status."""
    return load().nvfp4_group_gemm(problems, num_groups, stream)


def gemm_plan(M, N, K) -> dict:
    info = Nvfp4PlanInfo()
    _check(load().nvfp4_gemm_plan(M, N, K, ctypes.byref(info)))
    return info.as_dict()


def group_gemm_plan(shapes):
    """Plan for a list of (M, N, K): (info dict, tile prefix list)."""
    arr = (Nvfp4Problem * max(1, len(shapes)))()
    for i, (M, N, K) in enumerate(shapes):
        arr[i] = Nvfp4Problem(256, 256, 256, 256, 256, M, N, K)
    info = Nvfp4PlanInfo()
    prefix = (ctypes.c_int * (len(shapes) + 1))()
    _check(load().nvfp4_group_gemm_plan(arr, len(shapes), ctypes.byref(info), prefix))
    return info.as_dict(), list(prefix)


def release_workspaces():
    _check(load().nvfp4_release_workspaces())


def abi_version() -> int:
    return load().nvfp4_abi_version()
