"""MXFP8 storage of the saved pre-activation (test infrastructure only).

"Kimi K3 ... Memory" (section on the unified activation manager, and the closing summary
of the ledger) stores most saved activations block-wise in FP8, halving them again. The
pages give neither the element format nor the block size or scale type. The reading taken
here is the OCP Microscaling (MX) v1.0 format MXFP8 with E4M3 elements:

  * element E4M3: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no infinities;
    S.1111.111 is NaN; largest finite 1.75 * 2^8 = 448; smallest normal 2^-6; subnormal
    quantum 2^-9. Conversion rounds to nearest, ties to even, and saturates to +-448.
  * block: 32 consecutive elements along the last dimension share one scale 2^X, stored
    as an E8M0 byte X + 127.
  * X = floor(log2(amax)) - 8 (8 = exponent of E4M3's largest power of two, 256), clamped
    to [-127, 127]; a block of zeros takes X = -127. Elements are encoded from v / 2^X,
    so a block's largest magnitude lands in [256, 512) and values above 448 saturate.

Everything here is written from those definitions in fp64 (the division by 2^X is exact).
"""
import numpy as np

BLOCK = 32
EMAX_ELEM = 8
MAX_E4M3 = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """E4M3 byte -> fp64 value (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = c & 0x7
    val = np.where(ex == 0, man * 2.0 ** -9, (1.0 + man / 8.0) * np.ldexp(1.0, ex - 7))
    val = np.where((ex == 0xF) & (man == 0x7), np.nan, val)
    return sign * val


# the 127 non-negative finite values, ascending with their codes (code n <-> value n)
_POS = e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode(x) -> np.ndarray:
    """Finite fp64 -> nearest E4M3 byte, ties to the even code, saturating to +-448."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), MAX_E4M3)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 126)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(hi % 2 == 0, hi, lo)))
    pick = np.where(_POS[hi] == a, hi, pick)
    # the sign is kept, also when the magnitude rounds to zero (code 0x80)
    return (pick | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def block_scale_exp(amax) -> np.ndarray:
    """Shared exponent X of a block with largest magnitude amax (>= 0)."""
    amax = np.asarray(amax, dtype=np.float64)
    # floor(log2(amax)) from the binary exponent (amax = m 2^fe, 0.5 <= m < 1), exact
    _, fe = np.frexp(np.where(amax > 0, amax, 1.0))
    e = (fe - 1).astype(np.int64)
    X = np.clip(e - EMAX_ELEM, -127, 127)
    return np.where(amax > 0, X, -127).astype(np.int64)


def quantize(v, block=BLOCK):
    """v [..., n] (n a multiple of block) -> (codes uint8 [..., n], scale bytes uint8 [..., n/block])."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[-1]
    assert n % block == 0
    vb = v.reshape(v.shape[:-1] + (n // block, block))
    X = block_scale_exp(np.max(np.abs(vb), axis=-1))
    codes = e4m3_encode(vb / np.ldexp(1.0, X)[..., None])
    return codes.reshape(v.shape), (X + 127).astype(np.uint8)


def dequantize(codes, scales, block=BLOCK) -> np.ndarray:
    """Inverse of quantize (exact: E4M3 value times a power of two)."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    X = np.asarray(scales, dtype=np.int64) - 127
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (n // block, block))
    return (vals * np.ldexp(1.0, X)[..., None]).reshape(codes.shape)


def roundtrip(v, block=BLOCK) -> np.ndarray:
    """The value the backward sees for a stored v."""
    c, s = quantize(v, block)
    return dequantize(c, s, block)
