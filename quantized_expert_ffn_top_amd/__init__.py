"""Routed, block-quantized MoE FFN layer on AMD Instinct MI355X (gfx950).

The layer runs in libmoe.so (HIP kernels behind the C ABI of include/moe.h);
this package is its Python binding (ctypes) plus the build script.
"""

from ._lib import (EXPORTS, LIB_PATH, MOE_FMT_BF16, MOE_FMT_NL4_32, MOE_FMT_NL4S256, MOE_FMT_Q2_32,
                   MOE_FMT_Q2S256, MOE_FMT_Q3K256, MOE_FMT_Q3S256, MOE_PATH_BANDWIDTH, MOE_PATH_GEMM,
                   LayerDesc, LayerWeights, MoeError, desc, load, moe_combine, moe_dequantize,
                   moe_dequantize_path,
                   moe_expert_ffn, moe_layer_forward, moe_layer_forward_noalloc, moe_layer_forward_residual,
                   moe_layer_forward_timed,
                   moe_permute, moe_rmsnorm_residual,
                   moe_route, moe_router_logits, moe_workspace_size, weights, workspace)

__all__ = ["EXPORTS", "LIB_PATH", "MOE_FMT_BF16", "MOE_FMT_NL4_32", "MOE_FMT_Q2_32",
           "MOE_FMT_Q2S256", "MOE_FMT_Q3S256", "MOE_FMT_Q3K256", "MOE_FMT_NL4S256",
           "MOE_PATH_BANDWIDTH", "MOE_PATH_GEMM",
           "LayerDesc", "LayerWeights", "MoeError", "desc", "load", "moe_combine",
           "moe_dequantize", "moe_dequantize_path", "moe_expert_ffn", "moe_layer_forward", "moe_layer_forward_noalloc",
           "moe_layer_forward_residual",
           "moe_layer_forward_timed",
           "moe_permute",
           "moe_rmsnorm_residual", "moe_route", "moe_router_logits", "moe_workspace_size",
           "weights", "workspace"]
