"""Number formats used by the MoE layer, written out from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the formats but define none of them: the GC-MoE operator is an
"FP8/FP4" operator [GC-MoE feed, Full text] and MX block scaling gives each
32-element block one shared exponent [GC-MoE explainer, "Two MMA
Implementations in the Compute Partition"].  The encodings below are the plain
public definitions of those formats:

  e4m3 (OCP FP8 "E4M3FN"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
      infinities; S.1111.111 is NaN; largest finite 448; subnormals 2^-9 apart.
  e2m1 (OCP FP4): 1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
      0, 0.5, 1, 1.5, 2, 3, 4, 6.
  e8m0 (OCP MX scale): an unsigned biased exponent, value 2^(b-127); 255 is NaN.
  bf16: the upper half of an IEEE binary32; round to nearest, ties to even.

Everything here is exact dyadic arithmetic in fp64.
"""
import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code):
    """Value of one e4m3 code (0..255) as a Python float."""
    code = int(code)
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        mag = (man / 8.0) * 2.0 ** (1 - 7)          # subnormal: 0.m * 2^(1-bias)
    else:
        mag = (1.0 + man / 8.0) * 2.0 ** (exp - 7)  # normal: 1.m * 2^(e-bias)
    return sign * mag


# decode table built from the definition above, one entry per code
_E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_decode(codes):
    """uint8 array of e4m3 codes -> fp64 values."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x):
    """Round fp64/fp32 values to the nearest e4m3 code, ties to even mantissa.

    Magnitudes above 448 saturate to 448 (the method clamps before it encodes).
    The rounding is done on the exact value: within a binade [2^e, 2^(e+1)) the
    representable magnitudes are 2^(e-3) apart; below 2^-6 they are 2^-9 apart.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("e4m3_encode: NaN input")
    mag = np.minimum(np.abs(x), E4M3_MAX)
    # exponent of the binade holding mag, floored at the subnormal binade
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    e = np.maximum(e, -6.0)
    quantum = np.ldexp(1.0, (e - 3).astype(np.int64))
    steps = np.round(mag / quantum)          # numpy rounds halves to even
    q = steps * quantum
    q = np.minimum(q, E4M3_MAX)
    # map the exact magnitude back to its code through the decode table
    pos = _E4M3_TABLE[:127]
    idx = np.searchsorted(pos, q)
    if not np.all(pos[np.minimum(idx, 126)] == q):
        raise AssertionError("e4m3_encode: rounded value is not representable")
    code = idx.astype(np.uint8)
    neg = (x < 0) & (q > 0)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def e2m1_value(nib):
    """Value of one e2m1 nibble (0..15)."""
    nib = int(nib)
    sign = -1.0 if nib & 0x8 else 1.0
    exp = (nib >> 1) & 0x3
    man = nib & 0x1
    if exp == 0:
        mag = man * 0.5                           # subnormal: 0.m * 2^(1-bias)
    else:
        mag = (1.0 + man / 2.0) * 2.0 ** (exp - 1)
    return sign * mag


_E2M1_TABLE = np.array([e2m1_value(n) for n in range(16)], dtype=np.float64)


def e2m1_unpack(packed):
    """uint8 array [..., K/2] of packed FP4 pairs -> fp64 [..., K].

    Element 2i is the low nibble of byte i and element 2i+1 the high nibble
    (the OCP MX packing order).
    """
    packed = np.asarray(packed, dtype=np.uint8)
    lo = _E2M1_TABLE[packed & 0x0F]
    hi = _E2M1_TABLE[packed >> 4]
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def e8m0_decode(b):
    """uint8 e8m0 scale codes -> fp64 multipliers 2^(b-127); 255 -> NaN."""
    b = np.asarray(b, dtype=np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def bf16_round(x):
    """Round fp64 values to the nearest bf16 value (8 significand bits), ties to even.

    Returned as fp64.  Normal range only (the layer's outputs are far from the
    bf16 subnormal range); magnitudes that round past the largest bf16 become inf.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                 # x = m * 2^e, 0.5 <= |m| < 1
    r = np.round(m * 256.0)            # 8 significand bits, halves to even
    return np.ldexp(r, e - 8)


def bf16_decode(bits):
    """bf16 bit patterns (uint16) -> fp64 values: the top 16 bits of an IEEE fp32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def fp32_round(x):
    """Round fp64 values to the nearest fp32 value (IEEE round to nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
