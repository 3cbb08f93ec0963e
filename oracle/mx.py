"""MX codec and block quantizers (CPU oracle, test infrastructure only).

What the pages fix ([Blog], "Understanding OCP MXFP8 Microscaling on
Blackwell"): blocks of 32 contiguous elements share one 8-bit E8M0 scale
s = 2**(E8M0 - 127); each element is stored as an 8-bit FP8 value v_i, and the
block represents s * v_i.  The attention operands use E4M3 payloads
([Blog], "PyTorch Integration & Implementation Example": float8_e4m3fn).

What the pages leave open, and the reading taken (listed in the design notes):
  * E4M3 is the OCP "FN" variant: bias 7, no infinities, 0x7F/0xFF are NaN,
    largest finite 448, subnormals m * 2**-9.
  * Encoding rounds to nearest, ties to even, and saturates to +-448.
  * The scale is chosen from the block amax by the OCP MX rule:
    E8M0 = floor(log2(amax)) - 8 + 127 (8 = exponent of E4M3's largest power
    of two), clamped to [0, 254]; an all-zero block takes code 0.
  * floor(log2(.)) is read off the binary exponent (frexp), never a rounded log.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E8M0_BIAS = 127
E4M3_EMAX = 8
E4M3_MAX = 448.0


# ------------------------------------------------------------------ codecs
def e4m3_decode(codes) -> np.ndarray:
    """E4M3FN byte -> float64 (OCP FP8: sign | 4-bit exponent, bias 7 | 3-bit mantissa)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(y) -> np.ndarray:
    """float -> E4M3FN byte, round to nearest even, saturating at +-448.

    Subnormal range (|y| < 2**-6): the code is the integer RNE(|y| * 2**9) in
    [0, 8] (8 is the smallest normal, code 0x08).  Normal range: with
    e = floor(log2|y|), mantissa m = RNE((|y| / 2**e - 1) * 8); a carry m == 8
    moves to the next binade.  Anything beyond 448 saturates to code 0x7E.
    The sign bit is kept, so -0.0 encodes as 0x80.
    """
    y = np.asarray(y, dtype=np.float64)
    if np.any(np.isnan(y)):
        raise ValueError("e4m3_encode: NaN input is outside the oracle's contract")
    a = np.abs(y)
    neg = np.signbit(y)
    # subnormals and zero
    q_sub = np.rint(a * 2.0 ** 9)                      # exact scaling, RNE
    # normals
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(a)                            # a = f * 2**ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1                        # floor(log2 a)
    m = np.rint((np.ldexp(a, -e) - 1.0) * 8.0)         # exact until rint, RNE
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    normal_code = ((e + 7) << 3) | m.astype(np.int64)
    overflow = (e > 8) | ((e == 8) & (m == 7))
    normal_code = np.where(overflow, 0x7E, normal_code)
    code = np.where(a < 2.0 ** -6, q_sub.astype(np.int64), normal_code)
    code = np.where(np.isinf(a), 0x7E, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def e4m3_exponent(codes) -> np.ndarray:
    """Binary exponent of an E4M3FN code's significand: E - 7 for normals, -6 for
    subnormals and zero (the format's fixed subnormal exponent)."""
    E = (np.asarray(codes).astype(np.int64) >> 3) & 0xF
    return np.where(E == 0, -6, E - 7)


def e8m0_value(k) -> np.ndarray:
    """E8M0 byte -> 2**(k - 127) (255 is NaN)."""
    k = np.asarray(k).astype(np.int64)
    return np.where(k == 255, np.nan, np.exp2(k - float(E8M0_BIAS)))


def scale_code(amax) -> np.ndarray:
    """E8M0 code chosen from a block's amax: clamp(floor(log2 amax) - 8 + 127, 0, 254)."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, ex = np.frexp(amax)
    k = (ex.astype(np.int64) - 1) - E4M3_EMAX + E8M0_BIAS
    k = np.clip(k, 0, 254)
    return np.where(amax == 0, 0, k).astype(np.uint8)


# ------------------------------------------------------- block quantization
def quantize_blocks(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantize blocks laid out along the last axis (length 32).

    Returns (codes with x's shape, scale codes with the last axis dropped).
    Zero padding inside a block is harmless: it cannot raise the amax, and
    callers drop the codes it produces.
    """
    x = np.asarray(x, dtype=np.float64)
    assert x.shape[-1] == BLOCK
    amax = np.max(np.abs(x), axis=-1)
    k = scale_code(amax)
    y = x * np.exp2(E8M0_BIAS - k.astype(np.float64))[..., None]   # exact power-of-two scaling
    return e4m3_encode(y), k


def dequantize_blocks(codes, k) -> np.ndarray:
    return e4m3_decode(codes) * e8m0_value(k)[..., None]


def element_exponent_row32(codes, k):
    """Per-element exponent (E4M3 exponent + scale exponent) for ROW32 codes."""
    codes = np.asarray(codes)
    e = e4m3_exponent(codes)
    D = codes.shape[-1]
    ks = np.repeat(np.asarray(k).astype(np.int64) - E8M0_BIAS, BLOCK, axis=-1)[..., :D]
    return e + ks


def element_exponent_col32(codes, k, axis: int):
    ks = np.repeat(np.asarray(k).astype(np.int64) - E8M0_BIAS, BLOCK, axis=axis)
    ks = np.take(ks, np.arange(np.asarray(codes).shape[axis]), axis=axis)
    return e4m3_exponent(codes) + ks


def element_exponent_sq32(codes, k, axis_pos: int):
    ks = np.repeat(np.repeat(np.asarray(k).astype(np.int64) - E8M0_BIAS, BLOCK, axis=axis_pos), BLOCK, axis=-1)
    ks = np.take(ks, np.arange(np.asarray(codes).shape[axis_pos]), axis=axis_pos)
    ks = np.take(ks, np.arange(np.asarray(codes).shape[-1]), axis=-1)
    return e4m3_exponent(codes) + ks


def _pad_to(x: np.ndarray, axis: int, mult: int) -> np.ndarray:
    n = x.shape[axis]
    pad = (-n) % mult
    if pad == 0:
        return x
    widths = [(0, 0)] * x.ndim
    widths[axis] = (0, pad)
    return np.pad(x, widths)


def quantize_row32(x):
    """Blocks of 32 along the last (feature) axis.  x[..., D] -> codes[..., D], scales[..., D/32]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % BLOCK == 0
    codes, k = quantize_blocks(x.reshape(*x.shape[:-1], D // BLOCK, BLOCK))
    return codes.reshape(x.shape), k


def quantize_col32(x, axis: int):
    """Blocks of 32 consecutive positions along ``axis`` (aligned at 0; a short
    tail block holds the remaining positions).  Scales have ceil(n/32) entries
    along that axis."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[axis]
    xp = np.moveaxis(_pad_to(x, axis, BLOCK), axis, -1)          # [..., nb*32]
    nb = xp.shape[-1] // BLOCK
    codes, k = quantize_blocks(xp.reshape(*xp.shape[:-1], nb, BLOCK))
    codes = np.moveaxis(codes.reshape(xp.shape), -1, axis)
    codes = np.take(codes, np.arange(n), axis=axis)
    return codes, np.moveaxis(k, -1, axis)


def quantize_sq32(x, axis_pos: int):
    """Square [32 x 32] blocks over (positions along ``axis_pos``) x (last axis).

    Both axes are blocked from index 0; a short tail block along either axis
    holds the remaining entries.  Scales have ceil(n/32) entries along
    ``axis_pos`` and ceil(D/32) along the last axis.  The same codes come out
    whichever of the two axes is read as the contraction axis (transpose
    invariance, [News], forward/backward paragraph).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[axis_pos]
    D = x.shape[-1]
    assert 0 <= axis_pos < x.ndim - 1
    xp = np.moveaxis(_pad_to(_pad_to(x, axis_pos, BLOCK), x.ndim - 1, BLOCK), axis_pos, -2)
    nb, Dp = xp.shape[-2] // BLOCK, xp.shape[-1]
    blk = xp.reshape(*xp.shape[:-2], nb, BLOCK, Dp // BLOCK, BLOCK)
    blk = np.swapaxes(blk, -3, -2)                                 # [..., nb, Dp/32, 32, 32]
    flat = blk.reshape(*blk.shape[:-2], BLOCK * BLOCK)
    amax = np.max(np.abs(flat), axis=-1)
    k = scale_code(amax)
    y = flat * np.exp2(E8M0_BIAS - k.astype(np.float64))[..., None]
    codes = e4m3_encode(y).reshape(blk.shape)
    codes = np.swapaxes(codes, -3, -2).reshape(xp.shape)
    codes = np.moveaxis(codes, -2, axis_pos)
    codes = np.take(np.take(codes, np.arange(n), axis=axis_pos), np.arange(D), axis=-1)
    return codes, np.moveaxis(k, -2, axis_pos)


def dequantize_row32(codes, k):
    codes = np.asarray(codes)
    D = codes.shape[-1]
    v = dequantize_blocks(codes.reshape(*codes.shape[:-1], D // BLOCK, BLOCK), k)
    return v.reshape(codes.shape)


def dequantize_col32(codes, k, axis: int):
    scale = np.repeat(e8m0_value(k), BLOCK, axis=axis)
    scale = np.take(scale, np.arange(codes.shape[axis]), axis=axis)
    return e4m3_decode(codes) * scale


def dequantize_sq32(codes, k, axis_pos: int):
    scale = np.repeat(np.repeat(e8m0_value(k), BLOCK, axis=axis_pos), BLOCK, axis=-1)
    scale = np.take(scale, np.arange(codes.shape[axis_pos]), axis=axis_pos)
    scale = np.take(scale, np.arange(codes.shape[-1]), axis=-1)
    return e4m3_decode(codes) * scale


# ------------------------------------------------------------- varlen scales
def padded_offsets(seqlens, align: int = 128) -> np.ndarray:
    """Per-sequence scale-row offsets: prefix sum of lengths rounded up to 128
    ([News], contributions paragraph: scales of jagged tensors sit at padded,
    128-aligned addresses while the FP8 payload stays at its packed position)."""
    L = np.asarray(seqlens, dtype=np.int64)
    return np.concatenate([[0], np.cumsum((L + align - 1) // align * align)]).astype(np.int64)


def quantize_varlen(x, cu_seqlens, layouts=("row32", "col32", "sq32")):
    """Quantize a packed [T, H, D] tensor sequence by sequence.

    Payload codes stay at their packed token positions.  Scale tensors are
    indexed by padded offsets po_s (multiples of 128): ROW32 scales live at row
    po_s + t of [T_pad, H, D/32]; COL32 and SQ32 scales at row po_s/32 + t/32
    of [T_pad/32, H, D] and [T_pad/32, H, D/32].  Pad slots stay zero.
    Blocks along the sequence start at each sequence's first token.
    """
    x = np.asarray(x, dtype=np.float64)
    T, H, D = x.shape
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    L = np.diff(cu)
    po = padded_offsets(L)
    Tp = int(po[-1])
    out = {}
    for lay in layouts:
        codes = np.zeros((T, H, D), np.uint8)
        if lay == "row32":
            sc = np.zeros((Tp, H, D // BLOCK), np.uint8)
        elif lay == "col32":
            sc = np.zeros((Tp // BLOCK, H, D), np.uint8)
        else:
            sc = np.zeros((Tp // BLOCK, H, D // BLOCK), np.uint8)
        for s in range(len(L)):
            xs = x[cu[s]:cu[s + 1]]
            if len(xs) == 0:
                continue
            if lay == "row32":
                c, k = quantize_row32(xs)
                sc[po[s]:po[s] + len(xs)] = k
            elif lay == "col32":
                c, k = quantize_col32(xs, axis=0)
                sc[po[s] // BLOCK:po[s] // BLOCK + k.shape[0]] = k
            else:
                c, k = quantize_sq32(xs, axis_pos=0)
                sc[po[s] // BLOCK:po[s] // BLOCK + k.shape[0]] = k
            codes[cu[s]:cu[s + 1]] = c
        out[lay] = (codes, sc)
    return out


# ------------------------------------------------ admissible MX roundings
def element_magnitude(codes, k_elem):
    """2**(binade exponent) of each E4M3 element incl. its block scale (0 for zero codes); k_elem is
    the element's E8M0 code (already expanded to the codes' shape)."""
    codes = np.asarray(codes)
    e = e4m3_exponent(codes) + np.asarray(k_elem).astype(np.int64) - E8M0_BIAS
    return np.where((codes & 0x7F) != 0, np.exp2(e.astype(np.float64)), 0.0)


def block_max_2d(x, bq: int, bk: int):
    """Maximum of x [n, m] over blocks of bq rows x bk columns aligned at (0, 0) (short tail blocks)."""
    x = np.asarray(x, np.float64)
    n, m = x.shape
    xp = np.full(((n + bq - 1) // bq * bq, (m + bk - 1) // bk * bk), -np.inf)
    xp[:n, :m] = x
    return xp.reshape(xp.shape[0] // bq, bq, xp.shape[1] // bk, bk).max(axis=(1, 3))


def expand_2d(kb, bq: int, bk: int, shape):
    return np.repeat(np.repeat(np.asarray(kb), bq, axis=0), bk, axis=1)[:shape[0], :shape[1]]


def round_interval(lo, hi, bq: int, bk: int, floor_codes=(0, 1)):
    """MX rounding of a 2-D array known only up to intervals: each element lies anywhere in
    [lo, hi], blocks are bq x bk (aligned at (0, 0)), and each block's scale follows from its own
    (unknown) amax by the rule above.  Encoding is monotone in the value for a fixed scale, so the
    rounded value of an element lies between the smallest rounding of lo and the largest rounding of
    hi over the scale codes the block's amax interval allows.  ``floor_codes`` lists the smallest
    scale codes an implementation may substitute for code 0 (blocks whose amax is below 2^-118,
    whose contributions are below 2^-118 of the block's binade).  Returns (qlo, qhi, khi) with khi
    the largest admissible scale code per element."""
    lo = np.asarray(lo, np.float64)
    hi = np.asarray(hi, np.float64)
    alo = np.where(lo > 0, lo, np.where(hi < 0, -hi, 0.0))
    ahi = np.maximum(np.abs(lo), np.abs(hi))
    klo = expand_2d(scale_code(block_max_2d(alo, bq, bk)).astype(np.int64), bq, bk, lo.shape)
    khi = expand_2d(scale_code(block_max_2d(ahi, bq, bk)).astype(np.int64), bq, bk, lo.shape)
    qlo = np.full(lo.shape, np.inf)
    qhi = np.full(lo.shape, -np.inf)
    span = int(np.max(khi - klo)) if lo.size else 0
    for d in range(span + 1):
        k = np.minimum(klo + d, khi)
        for f in floor_codes:
            kk = np.maximum(k, f).astype(np.float64)
            s = np.exp2(kk - E8M0_BIAS)
            qlo = np.minimum(qlo, e4m3_decode(e4m3_encode(lo / s)) * s)
            qhi = np.maximum(qhi, e4m3_decode(e4m3_encode(hi / s)) * s)
    return qlo, qhi, np.maximum(khi, max(floor_codes))
