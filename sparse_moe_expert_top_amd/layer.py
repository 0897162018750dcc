"""The routed-expert layer (forward + backward) as a sequence of libmoe.so calls.

Forward ("Kimi K3 ... Memory", section "MoE 反向", forward equation; routing as in "Inside
Kimi K3", "Idea One"):
    moe_route_topk -> moe_permute -> moe_grouped_gemm_gate_up -> moe_grouped_gemm_down_combine
Saved for the backward: the pre-dispatch input x, the bf16 pre-activation h [R, 2H] and the
routing metadata; a and o are not kept ("Frontier-scale RL with Kimi K3", "Streaming
activations": only the bf16 input of the activation is saved).
Backward: moe_expert_bwd (re-dispatch, dA + SiTU-GLU' + dp, dW_down, dW_gu, dX, combine).
With h_store="mxfp8" the saved h is kept block-wise in FP8 instead ("Kimi K3 ... Memory",
unified activation manager: most saved activations are block-wise FP8), through
moe_grouped_gemm_gate_up_mx and moe_expert_bwd_mx.

W4A8 forward ("Frontier-scale RL with Kimi K3", "Low precision (MXFP4) rollouts": rollouts
run the MoE layers with 4-bit weights and 8-bit activations), forward only:
    moe_route_topk -> moe_permute -> moe_mxfp8_quantize(x) -> moe_grouped_gemm_gate_up_w4a8
    -> moe_grouped_gemm_down_combine_w4a8
with the weights quantized once to MXFP4 (`W4A8Weights`).

`LayerBuffers` allocates every buffer once (torch, HBM) so a training step issues only the
library's kernels; buffers indexed by routed rows are sized by a capacity R_cap (T*k by
default, which never overflows, or the exact routed rows of given logits), and the forward's
transients share their memory with the backward workspace.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import _lib


@dataclass
class LayerShape:
    T: int
    E: int
    k: int
    e_lo: int
    E_loc: int
    d: int
    H: int
    beta: float = 4.0
    linear_beta: float = 25.0


class W4A8Weights:
    """MXFP4 form of the expert weights for the W4A8 forward (quantized once, kept in HBM):
    gu codes [E_loc, 2H, d/2] + scales [E_loc, 2H, d/32], down codes [E_loc, d, H/2] + scales
    [E_loc, d, H/32], blocks along the reduction dimension."""

    def __init__(self, w_gu, w_down):
        E_loc, H2, d = w_gu.shape
        H = H2 // 2
        gq, gs = _lib.moe_mxfp4_quantize(w_gu.reshape(E_loc * H2, d))
        dq, ds = _lib.moe_mxfp4_quantize(w_down.reshape(E_loc * d, H))
        self.gu_codes = gq.view(E_loc, H2, d // 2)
        self.gu_scales = gs.view(E_loc, H2, d // 32)
        self.down_codes = dq.view(E_loc, d, H // 2)
        self.down_scales = ds.view(E_loc, d, H // 32)


def _round256(n: int) -> int:
    return (int(n) + 255) // 256 * 256


class LayerBuffers:
    """Device buffers for one layer call of a given shape, reused across steps.

    Row-indexed buffers are sized by the row capacity R_cap: T*k by default (never overflows),
    or the exact routed-row count of given logits (`routed_rows`). With alias=True the
    forward's transients (a and the down combine's fp32 rows) and the backward workspace share
    one arena: the forward's transients are dead once y is written, so the layer holds the
    saved h plus the larger of the two. combine_passes > 1 runs the forward's combine in that
    many passes over the output columns, shrinking its fp32 row buffer by that factor at the
    cost of re-reading the GEMM's row operand once per pass (results are bit-identical).
    bwd_passes does the same for the backward's dX combine. By default (None) it stays at
    combine_passes unless the backward's workspace would exceed the forward's share of the
    arena by 1 GiB or more; then it is the fewest passes whose workspace fits in that share,
    so the backward adds no memory beyond what the forward already needed. (At the
    large-context shapes that takes the peak from 69.9 to 60.0 GB for about 0.4 % of the step;
    at small shapes the extra pass costs more than the memory it saves.)"""

    def __init__(self, shape: LayerShape, R_cap: int | None = None, device="cuda",
                 h_store: str = "bf16", alias: bool = True, combine_passes: int = 1,
                 bwd_passes: int | None = None):
        if h_store not in ("bf16", "mxfp8"):
            raise ValueError(f"h_store must be 'bf16' or 'mxfp8', not {h_store!r}")
        s = shape
        self.shape = s
        self.h_store = h_store
        self.R_cap = s.T * s.k if R_cap is None else int(R_cap)
        self.combine_passes = int(combine_passes)
        R = max(self.R_cap, 1)
        i32, f32, bf, u8 = torch.int32, torch.float32, torch.bfloat16, torch.uint8
        e = lambda *sh, dt: torch.empty(sh, dtype=dt, device=device)
        self.topk_idx = e(s.T, s.k, dt=i32)
        self.gates = e(s.T, s.k, dt=f32)
        self.perm = dict(offsets=e(s.E_loc + 1, dt=i32), row_token=e(R, dt=i32),
                         row_gate=e(R, dt=f32), slot_row=e(s.T, s.k, dt=i32),
                         status=e(1, dt=i32))
        self.ws_perm = e(max(_lib.workspace_size(_lib.MOE_WS_PERMUTE, T=s.T, E_loc=s.E_loc), 256), dt=u8)
        if h_store == "mxfp8":
            self.h = None
            self.h_codes = e(R, 2 * s.H, dt=u8)
            self.h_scales = e(R, 2 * s.H // 32, dt=u8)
        else:
            self.h = e(R, 2 * s.H, dt=bf)
        sizes = dict(T=s.T, E_loc=s.E_loc, k=s.k, d=s.d, H=s.H, R_cap=self.R_cap)
        down_b = max(_lib.workspace_size_passes(_lib.MOE_WS_DOWN_COMBINE, self.combine_passes,
                                                **sizes), 256)
        a_b = _round256(R * s.H * 2)
        bwd_size = lambda p: max(_lib.workspace_size_passes(_lib.MOE_WS_EXPERT_BWD, p, **sizes), 256)
        if bwd_passes is None:
            bwd_passes = self.combine_passes
            if alias and bwd_size(bwd_passes) - (a_b + down_b) >= (1 << 30):
                max_p = max(1, s.d // 256)
                while bwd_passes < max_p and bwd_size(bwd_passes) > a_b + down_b:
                    bwd_passes += 1
        self.bwd_passes = int(bwd_passes)
        bwd_b = bwd_size(self.bwd_passes)
        if alias:
            self.arena = e(max(a_b + down_b, bwd_b), dt=u8)
            self.a = self.arena[:R * s.H * 2].view(bf).view(R, s.H)
            self.ws_down = self.arena[a_b:a_b + down_b]
            self.ws_bwd = self.arena[:bwd_b]
        else:
            self.arena = None
            self.a = e(R, s.H, dt=bf)
            self.ws_down = e(down_b, dt=u8)
            self.ws_bwd = e(bwd_b, dt=u8)
        self.y = e(s.T, s.d, dt=bf)
        self.dx = e(s.T, s.d, dt=bf)
        self.dw_gu = e(s.E_loc, 2 * s.H, s.d, dt=f32)
        self.dw_down = e(s.E_loc, s.d, s.H, dt=f32)
        self.dp = e(s.T, s.k, dt=f32)

    @staticmethod
    def routed_rows(shape: LayerShape, logits, device="cuda") -> int:
        """Local routed rows R of these logits (routes and permutes once with capacity T*k;
        reads 4 bytes back, so it synchronises). Sizing buffers at R_cap = R fits these logits
        exactly; other logits may route more rows (moe_permute then clamps and flags)."""
        s = shape
        idx, gates = _lib.moe_route_topk(logits, s.k)
        perm = _lib.moe_permute(idx, gates, s.e_lo, s.E_loc, s.T * s.k)
        return int(perm["offsets"][-1].item())

    # ------------------------------------------------------------------ steps
    def route(self, logits):
        s = self.shape
        _lib.moe_route_topk(logits, s.k, self.topk_idx, self.gates)
        _lib.moe_permute(self.topk_idx, self.gates, s.e_lo, s.E_loc, self.R_cap, out=self.perm,
                         ws=self.ws_perm)

    def gate_up(self, x, w_gu):
        """Gate/up GEMM with the SiTU-GLU epilogue: the saved h (bf16 or MXFP8) and a."""
        s = self.shape
        if self.h_store == "mxfp8":
            _lib.moe_grouped_gemm_gate_up_mx(x, self.perm["row_token"], self.perm["offsets"],
                                             w_gu, self.R_cap, s.beta, s.linear_beta,
                                             h_codes=self.h_codes, h_scales=self.h_scales,
                                             a=self.a)
        else:
            _lib.moe_grouped_gemm_gate_up(x, self.perm["row_token"], self.perm["offsets"], w_gu,
                                          self.R_cap, s.beta, s.linear_beta, h=self.h, a=self.a)

    def down_combine(self, w_down):
        """Down GEMM and combine into y."""
        _lib.moe_grouped_gemm_down_combine(self.a, self.perm["offsets"], self.perm["row_gate"],
                                           self.perm["slot_row"], w_down, self.R_cap, y=self.y,
                                           ws=self.ws_down)
        return self.y

    def forward(self, x, logits, w_gu, w_down):
        self.route(logits)
        self.gate_up(x, w_gu)
        return self.down_combine(w_down)

    def forward_w4a8(self, x, logits, w4: W4A8Weights):
        """W4A8 forward: x quantized to MXFP8 per token, a to MXFP8 per row; y in bf16."""
        s = self.shape
        if getattr(self, "x_codes", None) is None:
            dev = x.device
            R = max(self.R_cap, 1)
            self.x_codes = torch.empty((s.T, s.d), dtype=torch.uint8, device=dev)
            self.x_scales = torch.empty((s.T, s.d // 32), dtype=torch.uint8, device=dev)
            self.a_codes = torch.empty((R, s.H), dtype=torch.uint8, device=dev)
            self.a_scales = torch.empty((R, s.H // 32), dtype=torch.uint8, device=dev)
        self.route(logits)
        _lib.moe_mxfp8_quantize(x, codes=self.x_codes, scales=self.x_scales)
        _lib.moe_grouped_gemm_gate_up_w4a8(self.x_codes, self.x_scales, self.perm["row_token"],
                                           self.perm["offsets"], w4.gu_codes, w4.gu_scales,
                                           self.R_cap, s.beta, s.linear_beta,
                                           a_codes=self.a_codes, a_scales=self.a_scales)
        _lib.moe_grouped_gemm_down_combine_w4a8(self.a_codes, self.a_scales, self.perm["offsets"],
                                                self.perm["row_gate"], self.perm["slot_row"],
                                                w4.down_codes, w4.down_scales, self.R_cap,
                                                y=self.y, ws=self.ws_down)
        return self.y

    def backward(self, dy, x, w_gu, w_down, stages=_lib.MOE_BWD_ALL):
        """The backward, or the subset of its stages in `stages` (MOE_BWD_* bits; calls over
        one backward run the stages in their fixed order)."""
        s = self.shape
        hk = (dict(h_codes=self.h_codes, h_scales=self.h_scales) if self.h_store == "mxfp8"
              else dict(h=self.h))
        _lib.moe_expert_bwd_stages(dy, x, self.perm, w_gu, w_down, self.R_cap, stages, self.dx,
                                   self.dw_gu, self.dw_down, self.dp, self.ws_bwd,
                                   beta=s.beta, linear_beta=s.linear_beta, **hk)
        return self.dx, self.dw_gu, self.dw_down, self.dp

    def step(self, x, logits, w_gu, w_down, dy):
        """One forward + backward pass of the layer."""
        self.forward(x, logits, w_gu, w_down)
        return self.backward(dy, x, w_gu, w_down)

    def rows(self) -> int:
        """Routed local rows R (reads 4 bytes back from the device: synchronises)."""
        return int(self.perm["offsets"][-1].item())

    def overflowed(self) -> bool:
        return bool(self.perm["status"].item())
