"""MI355X-native NVFP4 block-scaled GEMM and grouped GEMM.

The computation lives in ``libnvfp4.so`` (hand-written HIP for gfx950 behind
the C ABI of include/nvfp4.h); this package is its thin Python binding.
"""
from ._binding import (  # noqa: F401
    Nvfp4Error,
    abi_version,
    gemm_plan,
    group_gemm_plan,
    load,
    nvfp4_gemm,
    nvfp4_group_gemm,
    release_workspaces,
    status_string,
)
