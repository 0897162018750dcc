"""W4A8 forward of the routed-expert layer in fp64 (test infrastructure only).

"Frontier-scale RL with Kimi K3", section "Low precision (MXFP4) rollouts": the rollout engine
runs the MoE layers with 4-bit weights and 8-bit activations (W4A8), forward only, with
everything outside the routed experts in bf16. The expert itself is the layer of
"Kimi K3 ... Memory", section "MoE 反向" (a_e = SiTU(W_gate x, W_up x), o_e = W_down a_e,
y = sum p_e o_e).

Readings (the pages fix neither formats nor where the quantizers sit):
  * weights are MXFP4 (`mxfp4`), blocked along the reduction dimension: w_gu[e] [2H, d]
    along d, w_down[e] [d, H] along H;
  * the 8-bit activations are MXFP8 E4M3 (`mxfp8`), blocked along the reduction dimension:
    the pre-dispatch input x per token along d, and the activation a per row along H;
  * between the two GEMMs the layer is the bf16 layer's: h = bf16(x8 . w4^T) and
    a = bf16(SiTU-GLU(h)); the down GEMM reads MXFP8(a); y = bf16(sum_e p_e o_e).
Every product of quantized values is exact in fp64; the sums are fp64.
"""
import numpy as np

from . import mxfp4, mxfp8
from .bf16 import bf16_round, bf16_widen
from .situ import situ_glu_fwd


def _f64(a):
    a = np.asarray(a)
    return bf16_widen(a) if a.dtype == np.uint16 else a.astype(np.float64)


def expert_layer_fwd_w4a8(x, w_gu, w_down, perm, H, beta=4.0, linear_beta=25.0):
    """Grouped W4A8 forward, one local expert at a time.

    x [T,d] (bf16 bits or float), w_gu [E_loc,2H,d], w_down [E_loc,d,H] (full precision;
    quantized here), perm from `permute`. Returns dict(y [T,d] bf16-rounded, y_sum [T,d] (the
    fp64 sum before that rounding), h [R,2H],
    a [R,H], a_codes [R,H], a_scales [R,H/32], h_mag [R,2H]) with h_mag = |x8| . |w4_gu|^T,
    the sum of the magnitudes of the products behind each h (a scale for error bounds). The
    MXFP8 blocks of x run along each token's row, so quantizing the gathered rows of an
    expert equals gathering the quantized x.
    """
    x = np.asarray(x)
    T, d = x.shape
    off, row_token, row_gate = perm["offsets"], perm["row_token"], perm["row_gate"]
    E_loc = len(off) - 1
    R = int(off[-1])
    y = np.zeros((T, d))
    h_all = np.zeros((R, 2 * H))
    h_mag = np.zeros((R, 2 * H))
    a_all = np.zeros((R, H))
    a_codes = np.zeros((R, H), np.uint8)
    a_scales = np.zeros((R, H // mxfp8.BLOCK), np.uint8)
    for e in range(E_loc):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        tok = row_token[r0:r1]
        x8 = mxfp8.roundtrip(_f64(x[tok]))
        wgu4 = mxfp4.roundtrip(_f64(w_gu[e]))
        wd4 = mxfp4.roundtrip(_f64(w_down[e]))
        h = bf16_round(x8 @ wgu4.T)
        a = bf16_round(situ_glu_fwd(h, H, beta, linear_beta))
        ac, asc = mxfp8.quantize(a)
        o = mxfp8.dequantize(ac, asc) @ wd4.T
        y[tok] += row_gate[r0:r1, None] * o      # a token occurs at most once per expert
        h_all[r0:r1], a_all[r0:r1] = h, a
        h_mag[r0:r1] = np.abs(x8) @ np.abs(wgu4).T
        a_codes[r0:r1], a_scales[r0:r1] = ac, asc
    return dict(y=bf16_round(y), y_sum=y, h=h_all, a=a_all, a_codes=a_codes,
                a_scales=a_scales, h_mag=h_mag)
