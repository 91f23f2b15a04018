"""Number formats of the oracle, written from their public definitions.

* BF16: the upper 16 bits of an IEEE-754 binary32.
* FP8 E4M3 ("e4m3fn", OCP 8-bit floating point): 1 sign bit, 4 exponent bits
  (bias 7), 3 mantissa bits; no infinities; S.1111.111 is NaN; largest finite
  magnitude 448 = 1.75 * 2^8; smallest normal 2^-6; subnormals m * 2^-9.
* E8M0 (OCP Microscaling v1.0 scale type): the value 2^(c - 127); c = 255 NaN.
* MX block quantization (OCP Microscaling v1.0), the reading of "MXFP8" taken
  for the MoK summary's MXFP8 forward ("What is 2.37x measured against"):
  blocks of 32 consecutive elements along the reduction dim share one E8M0
  scale 2^s with s = floor(log2(max |v|)) - 8 (8 = exponent of E4M3's largest
  binade), clamped to [-127, 127]; each element is v / 2^s rounded to the
  nearest E4M3 value, ties to even, saturating to +-448.  An all-zero block
  gets scale code 0 and all-zero codes.

Everything is float64 and exact: scaling by powers of two and the rounding
below introduce no error beyond the format's own rounding.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_E4M3_EMAX = 8          # exponent of the largest E4M3 binade
_E4M3_EMIN = -6         # exponent of the smallest normal


def bf16_decode(bits) -> np.ndarray:
    """uint16 BF16 bit patterns -> float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def bf16_round(v) -> np.ndarray:
    """float64 -> the nearest BF16 value (8 significant bits, float32's
    exponent range), ties to even, returned as float64.  Finite inputs whose
    rounded magnitude stays below 2^128."""
    v = np.asarray(v, dtype=np.float64)
    _, ex = np.frexp(v)                           # v = m * 2^ex, 0.5 <= |m| < 1
    q = np.exp2(np.maximum(ex - 8, -133).astype(np.float64))   # one unit in the 8th bit
    return np.rint(v / q) * q                     # exact: q is a power of two


def _e4m3_value(c: np.ndarray) -> np.ndarray:
    """The E4M3 definition, code by code: sign, 4-bit exponent (bias 7; 0 =
    subnormal, m * 2^-9), 3-bit mantissa; S.1111.111 is NaN."""
    c = np.asarray(c, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    mag = np.where(ex == 0, man * 2.0 ** -9,
                   (1.0 + man / 8.0) * np.exp2((ex - 7).astype(np.float64)))
    mag = np.where((ex == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


# the value of every one of the 256 codes, from the definition above
_E4M3_VALUES = _e4m3_value(np.arange(256))


def e4m3_decode(codes) -> np.ndarray:
    """uint8 E4M3 codes -> float64 (exact); 0x7F / 0xFF decode to NaN.  Each
    code is looked up among the 256 values the definition gives."""
    return _E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e8m0_decode(codes) -> np.ndarray:
    """uint8 E8M0 scale codes -> float64 2^(c-127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def e4m3_encode(v) -> np.ndarray:
    """float64 -> uint8 E4M3 code, round to nearest, ties to even, saturating
    to +-448.  Inputs must be finite.  -0.0 encodes as 0x80."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input")
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.minimum(np.abs(v), E4M3_MAX)
    # binade exponent of a: a = m * 2^ex, m in [0.5, 1)  ->  floor(log2 a) = ex - 1
    _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, _E4M3_EMIN)   # subnormals share 2^-6's step
    step = np.exp2((e - 3).astype(np.float64))             # spacing of the binade
    q = np.rint(a / step).astype(np.int64)                 # np.rint: ties to even
    # q counts steps in binade e: normals q in [8, 16], subnormals (e = -6) q in [0, 8]
    code = np.where(e == _E4M3_EMIN,
                    q,                                       # 0..8 (8 = smallest normal)
                    ((e + 7) << 3) + (q - 8))                # q = 16 rolls into the next binade
    code = np.where(a == 0.0, 0, code)
    return (code | sign).astype(np.uint8)


def mx_quantize(v, block: int = 32):
    """MX block quantization along the last axis.

    Returns (codes uint8 [..., K], scale codes uint8 [..., K/block])."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % block:
        raise ValueError(f"last dim {K} is not a multiple of {block}")
    if not np.all(np.isfinite(v)):
        raise ValueError("mx_quantize: non-finite input")
    blocks = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.max(np.abs(blocks), axis=-1)
    _, ex = np.frexp(amax)                        # floor(log2 amax) = ex - 1 for amax > 0
    s = ex.astype(np.int64) - 1 - _E4M3_EMAX
    s = np.where(amax == 0.0, -127, s)
    s = np.clip(s, -127, 127)
    scaled = blocks / np.exp2(s.astype(np.float64))[..., None]
    codes = e4m3_encode(scaled).reshape(v.shape)
    return codes, (s + 127).astype(np.uint8)


def mx_dequantize(codes, scales, block: int = 32) -> np.ndarray:
    """Inverse of ``mx_quantize``'s encoding: codes * 2^(scale - 127)."""
    c = e4m3_decode(codes)
    K = c.shape[-1]
    s = e8m0_decode(scales)
    return (c.reshape(c.shape[:-1] + (K // block, block)) * s[..., None]).reshape(c.shape)
