"""MI355X-native routed-expert layer (Kimi-K3-style MoE, forward + backward, SiTU-GLU).

The compute lives in libmoe.so (hand-written gfx950 HIP kernels behind the C ABI declared
in include/moe.h); this package is its ctypes binding plus buffer management in torch.
"""
from ._lib import (MoEError, load, workspace_size, workspace_size_passes, header_functions,
                   LIB_PATH, moe_route_topk, moe_permute, moe_unpermute,
                   moe_grouped_gemm_gate_up, situ_glu_fwd, situ_glu_bwd,
                   moe_grouped_gemm_down_combine, moe_expert_bwd, moe_expert_bwd_stages,
                   moe_router_bwd, moe_grouped_gemm_gate_up_mx, moe_expert_bwd_mx,
                   moe_mxfp8_quantize, moe_mxfp8_dequantize, moe_mxfp4_quantize,
                   moe_mxfp4_dequantize, moe_grouped_gemm_gate_up_w4a8,
                   moe_grouped_gemm_down_combine_w4a8, MOE_WS_PERMUTE, MOE_WS_SITU_GLU_FWD,
                   MOE_WS_SITU_GLU_BWD, MOE_WS_DOWN_COMBINE, MOE_WS_EXPERT_BWD, MOE_BWD_DA,
                   MOE_BWD_DW_DOWN, MOE_BWD_DW_GU, MOE_BWD_DX, MOE_BWD_DP, MOE_BWD_ALL)
from .layer import LayerShape, LayerBuffers, W4A8Weights

__all__ = [
    "MoEError", "load", "workspace_size", "workspace_size_passes", "header_functions",
    "LIB_PATH", "moe_route_topk", "moe_permute", "moe_unpermute", "moe_grouped_gemm_gate_up",
    "situ_glu_fwd", "situ_glu_bwd", "moe_grouped_gemm_down_combine", "moe_expert_bwd",
    "moe_expert_bwd_stages", "moe_router_bwd", "moe_grouped_gemm_gate_up_mx",
    "moe_expert_bwd_mx", "moe_mxfp8_quantize", "moe_mxfp8_dequantize", "moe_mxfp4_quantize",
    "moe_mxfp4_dequantize", "moe_grouped_gemm_gate_up_w4a8",
    "moe_grouped_gemm_down_combine_w4a8", "LayerShape", "LayerBuffers", "W4A8Weights",
    "MOE_WS_PERMUTE", "MOE_WS_SITU_GLU_FWD", "MOE_WS_SITU_GLU_BWD", "MOE_WS_DOWN_COMBINE",
    "MOE_WS_EXPERT_BWD", "MOE_BWD_DA", "MOE_BWD_DW_DOWN", "MOE_BWD_DW_GU", "MOE_BWD_DX",
    "MOE_BWD_DP", "MOE_BWD_ALL",
]
