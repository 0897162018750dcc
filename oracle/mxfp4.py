"""MXFP4 weights of the W4A8 expert forward (test infrastructure only).

"Frontier-scale RL with Kimi K3", section "Low precision (MXFP4) rollouts": the rollout engine
runs the MoE layers W4A8 (4-bit weights, 8-bit activations), everything else in bf16. The
explainer's "Idea Four" describes MXFP4 as a 4-bit float whose small blocks of weights share
one scale. Neither page fixes the element encoding, the block size or the scale type; the
reading taken here is OCP Microscaling (MX) v1.0 MXFP4:

  * element E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit; no infinities or
    NaN. Magnitudes 0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4, 6. Conversion rounds to
    nearest, ties to the even code, and saturates to +-6.
  * block: 32 consecutive elements along the last (reduction) dimension share one scale 2^X,
    stored as an E8M0 byte X + 127.
  * X = floor(log2(amax)) - 2 (2 = exponent of E2M1's largest power of two, 4), clamped to
    [-127, 127]; a block of zeros takes X = -127. Elements are encoded from v / 2^X, so a
    block's largest magnitude lands in [4, 8) and values above 6 saturate.

Storage (this library's reading; the format leaves packing open): a row of n elements is n/2
code bytes, element 2j in the low nibble of byte j and element 2j+1 in the high nibble, plus
n/32 scale bytes.

Everything is written from those definitions in fp64 (the division by 2^X is exact).
"""
import numpy as np

BLOCK = 32
EMAX_ELEM = 2
MAX_E2M1 = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """4-bit E2M1 code (0..15) -> fp64 value."""
    c = np.asarray(codes).astype(np.int64) & 0xF
    ex = (c >> 1) & 0x3
    man = c & 0x1
    mag = np.where(ex == 0, man * 0.5, (1.0 + man / 2.0) * np.ldexp(1.0, ex - 1))
    return np.where(c & 0x8, -mag, mag)


# the 8 non-negative values, ascending with their codes (code n <-> value n)
_POS = e2m1_decode(np.arange(8))


def e2m1_encode(x) -> np.ndarray:
    """Finite fp64 -> nearest E2M1 code (uint8 0..15), ties to the even code, saturating to +-6."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), MAX_E2M1)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 7)     # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(hi % 2 == 0, hi, lo)))
    pick = np.where(_POS[hi] == a, hi, pick)
    # the sign is kept, also when the magnitude rounds to zero (code 8)
    return (pick | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def block_scale_exp(amax) -> np.ndarray:
    """Shared exponent X of a block with largest magnitude amax (>= 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    _, fe = np.frexp(np.where(amax > 0, amax, 1.0))    # amax = m 2^fe, 0.5 <= m < 1
    X = np.clip((fe - 1).astype(np.int64) - EMAX_ELEM, -127, 127)
    return np.where(amax > 0, X, -127).astype(np.int64)


def pack(codes) -> np.ndarray:
    """[..., n] 4-bit codes -> [..., n/2] bytes, element 2j in the low nibble of byte j."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack(packed) -> np.ndarray:
    """Inverse of pack."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def quantize(v, block=BLOCK):
    """v [..., n] (n a multiple of block) -> (packed codes uint8 [..., n/2], scale bytes [..., n/block])."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    assert n % block == 0
    vb = v.reshape(v.shape[:-1] + (n // block, block))
    X = block_scale_exp(np.max(np.abs(vb), axis=-1))
    codes = e2m1_encode(vb / np.ldexp(1.0, X)[..., None]).reshape(v.shape)
    return pack(codes), (X + 127).astype(np.uint8)


def dequantize(packed, scales, block=BLOCK) -> np.ndarray:
    """Inverse of quantize (exact: an E2M1 value times a power of two)."""
    codes = unpack(packed)
    n = codes.shape[-1]
    X = np.asarray(scales, dtype=np.int64) - 127
    vals = e2m1_decode(codes).reshape(codes.shape[:-1] + (n // block, block))
    return (vals * np.ldexp(1.0, X)[..., None]).reshape(codes.shape)


def roundtrip(v, block=BLOCK) -> np.ndarray:
    """The value the W4A8 GEMM multiplies for a weight v."""
    c, s = quantize(v, block)
    return dequantize(c, s, block)
