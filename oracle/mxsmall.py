"""MXFP6 and MXFP4 element formats (CPU oracle, test infrastructure only).

The pages name MXFP6 and MXFP4 beside MXFP8 as the microscaling formats the
block-scaled MMA takes ([News], paragraph on Blackwell's block-scaled MMA
instructions).  They do not define them; the reading taken is the OCP
Microscaling (MX) v1.0 definition, the same family as MXFP8:

  * E2M3 (FP6): sign | 2-bit exponent, bias 1 | 3-bit mantissa; no Inf/NaN;
    largest 7.5, smallest normal 1, subnormals m/8.
  * E3M2 (FP6): sign | 3-bit exponent, bias 3 | 2-bit mantissa; no Inf/NaN;
    largest 28, smallest normal 0.25, subnormals m/16.
  * E2M1 (FP4): sign | 2-bit exponent, bias 1 | 1-bit mantissa; no Inf/NaN;
    values 0, 0.5, 1, 1.5, 2, 3, 4, 6.
  * Blocks of 32 along the contraction axis share one E8M0 scale, chosen by
    the OCP rule clamp(floor(log2 amax) - emax + 127, 0, 254) with emax the
    exponent of the format's largest power of two (2, 2 and 4 here, 8 for
    E4M3); encoding rounds to nearest, ties to even, and saturates.
  * Packing (the bitstream the matrix instruction reads, little-endian):
    element j of a row occupies bits [w j, w j + w) of the row's bytes, w = 4
    or 6 -- for FP4, element 2i in the low nibble of byte i.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E8M0_BIAS = 127

# name: (exponent bits, mantissa bits, bias, emax)
FORMATS = {
    "e2m3": (2, 3, 1, 2),
    "e3m2": (3, 2, 3, 4),
    "e2m1": (2, 1, 1, 2),
}
BITS = {"e2m3": 6, "e3m2": 6, "e2m1": 4}


def decode(codes, fmt: str) -> np.ndarray:
    """Element code -> float64."""
    eb, mb, bias, _ = FORMATS[fmt]
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> (eb + mb)) & 1, -1.0, 1.0)
    e = (c >> mb) & ((1 << eb) - 1)
    m = c & ((1 << mb) - 1)
    mag = np.where(e == 0, m * 2.0 ** (1 - bias - mb), (2**mb + m) * np.exp2(e - bias - mb))
    return sign * mag


def max_value(fmt: str) -> float:
    eb, mb, bias, _ = FORMATS[fmt]
    return float((2 ** (mb + 1) - 1) * 2.0 ** ((1 << eb) - 1 - bias - mb))


def encode(y, fmt: str) -> np.ndarray:
    """float -> code: round to nearest, ties to even, saturating at the format's max.

    With q = 2**(max(floor(log2|y|), 1 - bias) - mb) the spacing of the binade
    holding |y| (the subnormal spacing below the smallest normal), the value is
    RNE(|y| / q) * q; rounding up into the next binade stays representable,
    and anything above the largest value saturates.  The sign bit is kept.
    """
    eb, mb, bias, _ = FORMATS[fmt]
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.isnan(y)):
        raise ValueError("encode: NaN input is outside the oracle's contract")
    a = np.abs(y)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(a)
    e = np.maximum(ex.astype(np.int64) - 1, 1 - bias)          # binade, floored at the subnormal one
    r = np.rint(np.ldexp(a, mb - e))                           # |y| / q, RNE (exact scaling)
    r = np.where(np.isinf(a), np.inf, r)
    # r in [0, 2^(mb+1)]: r == 2^(mb+1) is the carry into the next binade
    carry = r >= 2 ** (mb + 1)
    e = np.where(carry, e + 1, e)
    r = np.where(carry, 2**mb, r)
    sub = r < 2**mb                                            # only possible in the lowest binade
    E = np.where(sub, 0, e + bias)
    M = np.where(sub, r, r - 2**mb)
    code = (E << mb) | M.astype(np.int64)
    top = ((1 << eb) - 1) << mb | ((1 << mb) - 1)              # largest finite code
    code = np.where((E > (1 << eb) - 1) | (a > max_value(fmt)), top, code)
    return (code | np.where(np.signbit(y), 1 << (eb + mb), 0)).astype(np.uint8)


def scale_code(amax, fmt: str) -> np.ndarray:
    """E8M0 code of a block: clamp(floor(log2 amax) - emax + 127, 0, 254); all-zero block -> 0."""
    emax = FORMATS[fmt][3]
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(amax)
    k = np.clip((ex.astype(np.int64) - 1) - emax + E8M0_BIAS, 0, 254)
    return np.where(amax == 0, 0, k).astype(np.uint8)


def quantize_rows(x, fmt: str):
    """Blocks of 32 along the last axis (its length a multiple of 32).
    Returns (codes, one per element, unpacked) and scale codes [..., n/32]."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n % BLOCK == 0
    xb = x.reshape(*x.shape[:-1], n // BLOCK, BLOCK)
    k = scale_code(np.max(np.abs(xb), axis=-1), fmt)
    y = xb * np.exp2(E8M0_BIAS - k.astype(np.float64))[..., None]   # exact power-of-two scaling
    return encode(y, fmt).reshape(x.shape), k


def dequantize_rows(codes, k, fmt: str) -> np.ndarray:
    codes = np.asarray(codes)
    n = codes.shape[-1]
    s = np.repeat(np.exp2(np.asarray(k).astype(np.float64) - E8M0_BIAS), BLOCK, axis=-1)[..., :n]
    return decode(codes, fmt) * s


def element_exponent_rows(codes, k, fmt: str) -> np.ndarray:
    """Binary exponent of each element's significand plus its scale exponent (the
    quantity the accumulation model groups by); subnormals and zero take 1 - bias."""
    eb, mb, bias, _ = FORMATS[fmt]
    codes = np.asarray(codes).astype(np.int64)
    E = (codes >> mb) & ((1 << eb) - 1)
    e = np.where(E == 0, 1 - bias, E - bias)
    n = codes.shape[-1]
    ks = np.repeat(np.asarray(k).astype(np.int64) - E8M0_BIAS, BLOCK, axis=-1)[..., :n]
    return e + ks


def pack(codes, fmt: str) -> np.ndarray:
    """Unpacked codes [..., n] -> bytes [..., n * w / 8], little-endian bitstream."""
    w = BITS[fmt]
    c = np.asarray(codes).astype(np.uint64)
    n = c.shape[-1]
    assert (n * w) % 8 == 0
    bits = ((c[..., :, None] >> np.arange(w, dtype=np.uint64)) & 1).reshape(*c.shape[:-1], n * w)
    by = bits.reshape(*c.shape[:-1], n * w // 8, 8)
    return (by << np.arange(8, dtype=np.uint64)).sum(axis=-1).astype(np.uint8)


def unpack(data, n: int, fmt: str) -> np.ndarray:
    w = BITS[fmt]
    d = np.asarray(data).astype(np.uint64)
    bits = ((d[..., :, None] >> np.arange(8, dtype=np.uint64)) & 1).reshape(*d.shape[:-1], -1)[..., :n * w]
    f = bits.reshape(*d.shape[:-1], n, w)
    return (f << np.arange(w, dtype=np.uint64)).sum(axis=-1).astype(np.uint8)


# ------------------------------------------------------------------ square blocks
def quantize_sq32(x, fmt: str):
    """Square [32 tokens x 32 features] blocks of a [L, D] head (Q, K in the backward with MXFP6 /
    MXFP4 operands: the backward's square blocks, [News] forward/backward paragraph, in the small
    element formats of the same paragraph family), blocked from (0, 0); a short tail block along the
    tokens holds the remaining rows.  Scale per block by this format's rule (scale_code).
    Returns (codes [L, D], one per element, unpacked) and scale codes [ceil(L/32), D/32]."""
    x = np.asarray(x, dtype=np.float64)
    L, D = x.shape
    assert D % BLOCK == 0
    nb = (L + BLOCK - 1) // BLOCK
    xp = np.zeros((nb * BLOCK, D))
    xp[:L] = x
    blk = xp.reshape(nb, BLOCK, D // BLOCK, BLOCK).swapaxes(1, 2)      # [nb, D/32, 32 tok, 32 feat]
    k = scale_code(np.max(np.abs(blk), axis=(2, 3)), fmt)
    y = blk * np.exp2(E8M0_BIAS - k.astype(np.float64))[:, :, None, None]
    codes = encode(y, fmt).swapaxes(1, 2).reshape(nb * BLOCK, D)[:L]
    return codes, k


def dequantize_sq32(codes, k, fmt: str) -> np.ndarray:
    codes = np.asarray(codes)
    L, D = codes.shape
    s = np.repeat(np.repeat(np.exp2(np.asarray(k).astype(np.float64) - E8M0_BIAS), BLOCK, axis=0), BLOCK, axis=1)
    return decode(codes, fmt) * s[:L, :D]


def element_exponent_sq32(codes, k, fmt: str) -> np.ndarray:
    """As element_exponent_rows, for square blocks."""
    eb, mb, bias, _ = FORMATS[fmt]
    codes = np.asarray(codes).astype(np.int64)
    L, D = codes.shape
    E = (codes >> mb) & ((1 << eb) - 1)
    e = np.where(E == 0, 1 - bias, E - bias)
    ks = np.repeat(np.repeat(np.asarray(k).astype(np.int64) - E8M0_BIAS, BLOCK, axis=0), BLOCK, axis=1)
    return e + ks[:L, :D]


def pack_sq32_columns(codes, fmt: str) -> np.ndarray:
    """The column-packed copy of square-block codes: for block row b and feature f, the 32 tokens
    32 b .. 32 b + 31 of column f as one packed block (tokens past L as code 0).  The instruction
    reads a transposed operand (contraction over tokens) as such blocks.  Returns bytes
    [ceil(L/32), D, 32 w / 8]."""
    codes = np.asarray(codes)
    L, D = codes.shape
    nb = (L + BLOCK - 1) // BLOCK
    cp = np.zeros((nb * BLOCK, D), dtype=np.uint8)
    cp[:L] = codes
    cols = cp.reshape(nb, BLOCK, D).swapaxes(1, 2)                      # [nb, D, 32 tokens]
    return pack(cols, fmt)
