"""fp64 CPU oracle for the routed-expert layer (forward and backward) and SiTU-GLU.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or links this package:
only the tests, the smoke check and the benchmark's CPU-baseline leg may use it. It shares
no code with the HIP library (no kernels, headers, helpers or tables); the only thing both
sides consume is the seeded input generator, which holds none of the layer's arithmetic.

What it computes, and where the pages define it:
  * routing (`route.route_topk`) - "Inside Kimi K3", "Idea One" routing snippet: top-k of the
    router scores, softmax over the k kept values.
  * dispatch metadata (`permute.permute`) - "Kimi K3 ... Memory", "MoE 反向" (second saving):
    the grouped GEMM reads a copy of the tokens sorted by expert.
  * SiTU-GLU (`situ`) - "Frontier-scale RL with Kimi K3", "Streaming activations": the naive
    activation's definition (gate half first, gate' = beta tanh(g/beta) sigmoid(g),
    lin' = lambda tanh(l/lambda), product, cast to the input dtype).
  * expert layer forward/backward (`layer`) - "Kimi K3 ... Memory", "MoE 反向": the expert
    forward equations (a_e, o_e, y) and the router-probability gradient rewritten as
    <W_down^T dL/dy, a_e> so o_e is never needed.
  * MXFP8 storage of the saved pre-activation (`mxfp8`) - "Kimi K3 ... Memory" (unified
    activation manager; ledger summary): saved activations kept block-wise in FP8. Format
    read as OCP MX v1.0 MXFP8 (E4M3 elements, 32-element blocks, E8M0 scales); the layer
    backward takes h_store="mxfp8" to recompute from the stored value.
  * W4A8 forward (`w4a8.expert_layer_fwd_w4a8`) with MXFP4 weights (`mxfp4`) - "Frontier-scale
    RL with Kimi K3", "Low precision (MXFP4) rollouts": rollouts run the MoE layers with
    4-bit weights and 8-bit activations. Formats read as OCP MX v1.0 MXFP4 (E2M1) and MXFP8
    (E4M3), blocks of 32 along the reduction dimension.

Two numeric modes:
  * "X" (exact): no intermediate rounding; used for the mathematical invariants.
  * "S" (storage-faithful): rounds fp64 -> bf16 (nearest-even, directly from fp64) exactly
    where the layer stores a bf16 tensor: h (saved pre-activation), a (activation output),
    dh, and the bf16 outputs y and dx. GPU parity is graded against mode S.

Parity status: every function here is pinned by tests under tests/ (closed forms, limits,
library special cases, brute force, finite differences, autograd). None is "parity unpinned".
"""
from .bf16 import bf16_round, bf16_widen
from .situ import situ_glu_fwd, situ_glu_bwd, situ_parts
from .route import route_topk
from .permute import permute
from . import mxfp4, mxfp8, w4a8
from .layer import (expert_layer_fwd, expert_layer_bwd, token_layer_fwd, token_layer_bwd,
                    dw_columns, router_bwd, unpermute_sum)

__all__ = [
    "bf16_round", "bf16_widen", "situ_glu_fwd", "situ_glu_bwd", "situ_parts",
    "route_topk", "permute", "expert_layer_fwd", "expert_layer_bwd", "token_layer_fwd",
    "token_layer_bwd", "dw_columns", "router_bwd", "unpermute_sum",
]
