"""One MI355X's share of an expert-parallel MoE layer: rank-major dispatch, FP8/MXFP4
block-scaled grouped GEMM with fused SwiGLU, and top-k-weighted combine.

The compute path is the HIP library `libctg_moe.so` (C-ABI declared in
include/ctg_moe.h); `binding` marshals arguments to it.  `synth` builds seeded
synthetic inputs.
"""
