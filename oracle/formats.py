"""Decoding of the stored number formats into float64 (test infrastructure).

The attention inputs are stored as bfloat16 (q, and K/V in the bf16 cache) or as
8-bit OCP E4M3 codes with float32 per-token-per-head scales (the FP8 KV cache that
page 2's roadmap and page 3's support section speak of). The oracle reads the exact
stored values: each code is turned into the real number it denotes, in float64.

Both decoders are written from the formats' definitions:

* bfloat16 is the upper half of an IEEE-754 binary32 word (1 sign, 8 exponent and 7
  fraction bits), so a code c denotes the binary32 number whose bits are ``c << 16``.
* OCP 8-bit floating point, E4M3 ("e4m3fn"): 1 sign bit, 4 exponent bits with bias 7,
  3 fraction bits. Exponent field 0 gives subnormals ``(m/8) * 2**-6``; otherwise the
  value is ``(1 + m/8) * 2**(e-7)``. There are no infinities; the two codes with all
  exponent and fraction bits set (0x7F, 0xFF) are NaN, so the largest finite magnitude
  is ``1.75 * 2**8 = 448``.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Return the float64 values of bfloat16 codes given as a uint16 array."""
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("bfloat16 codes must be uint16, got %s" % bits.dtype)
    words = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return words.view(np.float32).astype(np.float64)


def e4m3fn_codes_to_f64(codes):
    """Return the float64 values of OCP E4M3 codes given as a uint8 array."""
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8, got %s" % codes.dtype)
    c = codes.astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    subnormal = m / 8.0 * 2.0 ** -6
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    mag = np.where(e == 0, subnormal, normal)
    out = sign * mag
    out = np.where((c & 0x7F) == 0x7F, np.nan, out)
    return out
