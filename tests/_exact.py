"""Exact-rational brute-force references used to pin the oracle's codecs.

These are deliberately a different method from the oracle's: every E4M3 value
is enumerated as a Fraction and the nearest one is found by search; the MX
scale exponent is found by stepping powers of two, not by frexp.
"""
from __future__ import annotations

import bisect
import struct
from fractions import Fraction


def _e4m3_table():
    vals = []
    for code in range(0x7F):                 # 0x00 .. 0x7E: every finite magnitude
        ex, man = code >> 3, code & 7
        if ex == 0:
            v = Fraction(man, 512)           # subnormal: man * 2^-9
        else:
            v = (1 + Fraction(man, 8)) * Fraction(2) ** (ex - 7)
        vals.append((v, code))
    vals.sort()
    return vals


E4M3_TABLE = _e4m3_table()
_E4M3_VALUES = [v for v, _ in E4M3_TABLE]
E4M3_MAXF = Fraction(448)


def e4m3_nearest_code(x) -> int:
    """Nearest finite E4M3 code to the rational x, ties to the even code,
    magnitudes above 448 saturate.  Sign bit copied from x (so -0 -> 0x80)."""
    xf = Fraction(x)
    neg = xf < 0 or (xf == 0 and isinstance(x, float) and struct.pack(">d", x)[0] & 0x80)
    a = abs(xf)
    if a >= E4M3_MAXF:
        code = 0x7E
    else:
        i = bisect.bisect_left(_E4M3_VALUES, a)
        if i < len(_E4M3_VALUES) and _E4M3_VALUES[i] == a:
            code = E4M3_TABLE[i][1]
        else:
            lo_v, lo_c = E4M3_TABLE[i - 1]
            hi_v, hi_c = E4M3_TABLE[i]
            dlo, dhi = a - lo_v, hi_v - a
            if dlo < dhi:
                code = lo_c
            elif dhi < dlo:
                code = hi_c
            else:
                code = lo_c if lo_c % 2 == 0 else hi_c
    return code | (0x80 if neg else 0)


def mx_block_exact(block):
    """MX quantization of one block of floats, exactly: returns (codes, scale code)."""
    fr = [Fraction(v) for v in block]
    amax = max(abs(v) for v in fr)
    if amax == 0:
        s = -127
    else:
        # largest s with 2^(s+8) <= amax, i.e. s = floor(log2 amax) - 8
        s = 0
        while Fraction(2) ** (s + 8) > amax:
            s -= 1
        while Fraction(2) ** (s + 9) <= amax:
            s += 1
        s = max(-127, min(127, s))
    scale = Fraction(2) ** s
    codes = []
    for v, f in zip(block, fr):
        q = f / scale
        codes.append(e4m3_nearest_code(q) if q != 0 else e4m3_nearest_code(float(v)))
    return codes, s + 127


def bf16_bits_to_float(bits: int) -> float:
    """BF16 bits -> Python float through the binary32 byte layout."""
    return struct.unpack(">f", struct.pack(">I", (int(bits) & 0xFFFF) << 16))[0]
