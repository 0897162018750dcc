"""SiTU-GLU forward and backward in fp64 (test infrastructure only).

Definition ("Frontier-scale RL with Kimi K3", section "Streaming activations", the naive
activation): the input's last dimension splits into two halves, gate first and linear
second; gate' = beta * tanh(gate / beta) * sigmoid(gate) with beta = 4 by default,
lin' = linear_beta * tanh(linear / linear_beta) with linear_beta = 25 by default; the
output is gate' * lin', computed in fp32 from the widened input and cast back to the input
dtype. The oracle computes in fp64 and leaves any cast to the caller.

Backward (the custom op of the same section keeps only the bf16 input and recomputes tanh
and sigmoid): with t1 = tanh(g/beta), s = sigmoid(g), t2 = tanh(l/linear_beta),
  d gate'/dg = (1 - t1^2) s + beta t1 s (1 - s),     d lin'/dl = 1 - t2^2,
  dh = [ da * lin' * dgate'/dg ,  da * gate' * dlin'/dl ].
"""
import numpy as np
from scipy.special import expit


def situ_parts(h, H, beta=4.0, linear_beta=25.0):
    """Return (g, l, t1, s, t2, gate', lin') for h of shape [..., 2H] in fp64."""
    h = np.asarray(h, dtype=np.float64)
    assert h.shape[-1] == 2 * H, (h.shape, H)
    g = h[..., :H]
    l = h[..., H:]
    t1 = np.tanh(g / beta)
    s = expit(g)
    t2 = np.tanh(l / linear_beta)
    gate = beta * t1 * s
    lin = linear_beta * t2
    return g, l, t1, s, t2, gate, lin


def situ_glu_fwd(h, H, beta=4.0, linear_beta=25.0):
    """a = gate'(g) * lin'(l) for h = [g | l] of shape [..., 2H]; fp64 result [..., H]."""
    _, _, _, _, _, gate, lin = situ_parts(h, H, beta, linear_beta)
    return gate * lin


def situ_glu_bwd(h, da, H, beta=4.0, linear_beta=25.0):
    """dL/dh [..., 2H] given h [..., 2H] and dL/da [..., H], recomputing tanh and sigmoid."""
    da = np.asarray(da, dtype=np.float64)
    _, _, t1, s, t2, gate, lin = situ_parts(h, H, beta, linear_beta)
    dgate = (1.0 - t1 * t1) * s + beta * t1 * s * (1.0 - s)
    dlin = 1.0 - t2 * t2
    return np.concatenate([da * lin * dgate, da * gate * dlin], axis=-1)
