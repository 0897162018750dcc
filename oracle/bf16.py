"""bfloat16 storage semantics for the oracle (test infrastructure only).

The pages store the activation output with `.to(x.dtype)` from fp32 and call the saved
pre-activation "a bf16 [R, 2H] tensor" ("Frontier-scale RL with Kimi K3", "Streaming
activations"). They do not state a rounding mode; the reading taken here is PyTorch's
round-to-nearest-even. The oracle rounds directly from fp64 (no double rounding via fp32).

bfloat16: 1 sign bit, 8 exponent bits (same range as fp32), 7 stored mantissa bits, so a
normal value has 8 significant bits and the subnormal quantum is 2^-133.
"""
import numpy as np

_MAX_FINITE = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_round(v) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value (ties to even); return fp64."""
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    flat = v.reshape(-1)
    of = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat.size, step):
        x = flat[s:s + step]
        _, e = np.frexp(x)                       # x = m 2^e, 0.5 <= |m| < 1
        e = np.maximum(e, -125)                  # below 2^-126 the quantum stays 2^-133
        q = np.ldexp(1.0, e - 8)                 # 8 significant bits
        r = np.round(x / q) * q                  # np.round is round-half-to-even; x/q is exact
        r = np.where(np.abs(r) > _MAX_FINITE, np.copysign(np.inf, x), r)
        r = np.where(np.isfinite(x), r, x)
        of[s:s + step] = r
    return out


def bf16_widen(bits) -> np.ndarray:
    """Exact fp64 value of bf16 bit patterns given as uint16."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
