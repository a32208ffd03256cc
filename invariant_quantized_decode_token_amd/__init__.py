"""Batch-invariant int8 linear layer for decode and speculative-verify passes
on AMD Instinct MI355X (gfx950).

The computation lives in libiqd.so (hand-written HIP kernels behind the C ABI
of include/iqd.h); this package is its Python binding, with the same names.
"""
from ._lib import (IQD_K_MAX, IQD_OP_BLOCKQ8, IQD_OP_FP8, IQD_OP_KQ4, IQD_OP_KQ6, IQD_OP_LM_HEAD, IQD_OP_W8A8, IQD_OP_W8A8_BF16,
                   IQD_SPLIT_K_MAX, fp8_linear, kq4_linear, kq6_linear, quantize_fp8,
                   IqdError, attn_decode, attn_workspace_bytes, blockq8_linear, header_functions, lm_head_argmax, lm_head_argmax_static, load, pow2_requantize,
                   quantize_activations, read_ceiling, status_str, w8a8_linear, w8a8_linear_bf16, workspace_bytes)

__all__ = ["quantize_activations", "w8a8_linear", "w8a8_linear_bf16", "blockq8_linear", "lm_head_argmax", "lm_head_argmax_static",
           "quantize_fp8", "fp8_linear", "IQD_OP_FP8", "kq6_linear", "IQD_OP_KQ6", "kq4_linear", "IQD_OP_KQ4",
           "pow2_requantize", "read_ceiling", "attn_decode", "attn_workspace_bytes", "workspace_bytes", "status_str", "load", "header_functions", "IqdError", "IQD_K_MAX",
           "IQD_SPLIT_K_MAX", "IQD_OP_W8A8", "IQD_OP_BLOCKQ8", "IQD_OP_LM_HEAD", "IQD_OP_W8A8_BF16"]
