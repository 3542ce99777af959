"""MI355X-native NVFP4 block-scaled GEMM and grouped GEMM.

The computation lives in ``libnvfp4.so`` (hand-written HIP for gfx950 behind
the C ABI of include/nvfp4.h); this package is its thin Python binding.
"""
from ._binding import (  # noqa: F401
    NVFP4_MAX_GROUPS,
    NVFP4_MAX_K,
    Nvfp4Error,
    abi_version,
    gemm_plan,
    group_gemm_plan,
    load,
    nvfp4_blocked_scale_bytes,
    nvfp4_gemm,
    nvfp4_gemm_batched,
    nvfp4_gemm_blocked,
    nvfp4_gemm_noalloc,
    nvfp4_gemm_pow2scale,
    nvfp4_group_gemm,
    nvfp4_group_gemm_blocked,
    nvfp4_group_gemm_device,
    nvfp4_group_gemm_device_workspace_bytes,
    nvfp4_group_gemm_pow2scale,
    nvfp4_scales_from_blocked,
    nvfp4_scales_to_blocked,
    problem_table_bytes,
    release_workspaces,
    status_string,
)
