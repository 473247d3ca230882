"""Pyramid Sparse Attention path for AMD Instinct MI355X (gfx950): pyramid, mask, attention
forward and backward.

The compute lives in libpsa.so (HIP kernels behind the C ABI of include/psa.h); this package
is its ctypes binding. Build the library with `python -m video_transformers_amd.build`.
"""
from .psa import (EXPORTS, LIB_PATH, MaskParams, Problem, PsaError, attn_bwd, attn_bwd_workspace,
                  attn_fwd, attn_fwd_noalloc, attn_fwd_fp8, attn_fwd_fp8qk, attn_fwd_indexed, attn_fwd_meankey, attn_fwd_unpacked, attn_workspace,
                  build_index, build_pyramid, check_status, debug_fill_lds, forward, lib,
                  make_problem, mask, mask_assign, pooled_rows, quantize_fp8)

__all__ = ["EXPORTS", "LIB_PATH", "MaskParams", "Problem", "PsaError", "attn_bwd",
           "attn_bwd_workspace", "attn_fwd", "attn_fwd_noalloc", "attn_fwd_fp8", "attn_fwd_fp8qk", "attn_fwd_indexed", "attn_fwd_meankey",
           "attn_fwd_unpacked", "attn_workspace", "build_index", "build_pyramid", "check_status",
           "debug_fill_lds",
           "forward", "lib", "make_problem", "mask", "mask_assign", "pooled_rows", "quantize_fp8"]
