"""fp64 reference codecs for the three narrow formats of the CSA2 cache.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The report digest ("DeepSeek-V4.1-Flash", section 2.4.4) stores the main KV
as E2M1 elements with one E4M3 scale per 16 channels (NVFP4 without its
second-level scale) and the indexer K as OCP MXFP4 (E2M1 elements, one E8M0
scale per 32).  Its bound 448 x 6 = 2688 fixes the E4M3 flavour as OCP E4M3FN
(largest finite 448).  The bit layouts below are the OCP specifications':

  E2M1   s | e1 e0 | m        bias 1, no inf/NaN
         e == 0: (-1)^s * m * 0.5          (subnormal: 0 or 0.5)
         e  > 0: (-1)^s * (1 + m/2) * 2^(e-1)
  E4M3FN s | e3..e0 | m2..m0  bias 7, no inf, S.1111.111 is NaN
         e == 0: (-1)^s * m/8 * 2^-6
         e  > 0: (-1)^s * (1 + m/8) * 2^(e-7)
  E8M0   e7..e0               2^(e-127), 0xFF is NaN

Encoders round to nearest, ties to the code with an even mantissa (its low
bit clear), and saturate at the largest finite magnitude.  They are written
as an exhaustive nearest-value search over the decoded table, which is slow
and obviously right.
"""

import numpy as np


# ---------------------------------------------------------------- decoders
def e2m1_value(code):
    """Decode E2M1 nibbles (array of ints 0..15) to fp64."""
    c = np.asarray(code).astype(np.int64)
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def e4m3fn_value(code):
    """Decode OCP E4M3FN bytes to fp64; 0x7F / 0xFF decode to NaN."""
    c = np.asarray(code).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e8m0_value(code):
    """Decode E8M0 scale bytes to fp64 powers of two; 0xFF decodes to NaN."""
    c = np.asarray(code).astype(np.int64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


# ---------------------------------------------------------------- encoders
def _nearest_code(v, codes, values):
    """Round each |v| to the nearest of `values` (non-negative, ascending,
    paired with `codes`); ties go to the even code; beyond the largest value
    saturate to it."""
    v = np.asarray(v, dtype=np.float64)
    flat = np.abs(v).reshape(-1)
    out = np.empty(flat.shape, dtype=np.int64)
    even = ((codes & 1) == 0).reshape(1, -1)
    step = 1 << 15
    for i in range(0, flat.size, step):            # chunked only to bound memory
        a = flat[i:i + step].reshape(-1, 1)
        d = np.abs(a - values.reshape(1, -1))
        cand = d == d.min(axis=1, keepdims=True)
        # among equidistant candidates prefer the even code
        pick_even = cand & even
        has_even = pick_even.any(axis=1)
        idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
        out[i:i + step] = codes[idx]
    return out.reshape(v.shape)


_E2M1_POS_CODES = np.arange(8, dtype=np.int64)
_E2M1_POS_VALUES = e2m1_value(_E2M1_POS_CODES)

_E4M3_POS_CODES = np.arange(0x7F, dtype=np.int64)  # 0x00..0x7E, all finite
_E4M3_POS_VALUES = e4m3fn_value(_E4M3_POS_CODES)


def e2m1_encode(v):
    """fp64 -> E2M1 nibble, RNE, saturating at 6.  The sign bit is set iff
    v < 0, so a negative value that rounds to zero gives code 0x8 (-0)."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_code(v, _E2M1_POS_CODES, _E2M1_POS_VALUES)
    return (mag | np.where(v < 0, 8, 0)).astype(np.uint8)


def e4m3fn_encode(v):
    """fp64 -> E4M3FN byte, RNE, saturating at 448.  Sign bit set iff v < 0."""
    v = np.asarray(v, dtype=np.float64)
    mag = _nearest_code(v, _E4M3_POS_CODES, _E4M3_POS_VALUES)
    return (mag | np.where(v < 0, 0x80, 0)).astype(np.uint8)


# ---------------------------------------------------------------- packing
def pack_nibbles(codes):
    """[..., 2n] nibbles -> [..., n] bytes, channel 2c in the low nibble."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def unpack_nibbles(packed):
    """[..., n] bytes -> [..., 2n] nibbles, low nibble first."""
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
