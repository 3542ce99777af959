"""MI355X-native NVFP4 block-scaled GEMM and grouped GEMM."""
