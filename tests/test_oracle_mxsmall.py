"""Pins of the MXFP6 / MXFP4 codec (oracle/mxsmall.py) against the OCP MX
format definitions and brute force, independent of any kernel."""
import math

import numpy as np
import pytest

from oracle import mxsmall as ms

# facts of the OCP MX v1.0 element formats: (largest, smallest normal, smallest subnormal, #codes)
SPEC = {"e2m3": (7.5, 1.0, 0.125, 64), "e3m2": (28.0, 0.25, 0.0625, 64), "e2m1": (6.0, 1.0, 0.5, 16)}


@pytest.mark.parametrize("fmt", list(SPEC))
def test_decode_table_matches_the_format_facts(fmt):
    mx_, mn, sub, n = SPEC[fmt]
    v = ms.decode(np.arange(n), fmt)
    pos = v[: n // 2]
    assert np.all(np.diff(pos) > 0), "codes of one sign increase with the value"
    assert pos[0] == 0 and pos[1] == sub and pos[-1] == mx_ == ms.max_value(fmt)
    assert np.min(pos[pos >= mn]) == mn and np.all(np.isin(mn, pos))
    assert np.array_equal(v[n // 2:], -pos)                       # sign bit mirrors
    if fmt == "e2m1":
        assert pos.tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


@pytest.mark.parametrize("fmt", list(SPEC))
def test_encode_is_nearest_with_ties_to_even_and_saturates(fmt):
    n = SPEC[fmt][3]
    vals = ms.decode(np.arange(n // 2), fmt)
    rng = np.random.default_rng(0)
    y = np.concatenate([rng.uniform(-1.3, 1.3, 4000) * ms.max_value(fmt),
                        (vals[1:] + vals[:-1]) / 2, -(vals[1:] + vals[:-1]) / 2,    # exact ties
                        vals, -vals, [1e9, -1e9, 0.0]])
    got = ms.encode(y, fmt)
    a = np.minimum(np.abs(y), ms.max_value(fmt))
    d = np.abs(vals[None, :] - a[:, None])
    best = d == d.min(axis=1, keepdims=True)
    # among equally near codes take the even one (ties to even mantissa)
    cand = [np.flatnonzero(b) for b in best]
    want = np.array([c[0] if len(c) == 1 else c[c % 2 == 0][0] for c in cand])
    assert np.array_equal(got & (n // 2 - 1), want)
    assert np.array_equal(got >= n // 2, np.signbit(y))


@pytest.mark.parametrize("fmt", list(SPEC))
def test_scale_rule_puts_the_block_max_in_the_top_binade(fmt):
    emax = ms.FORMATS[fmt][3]
    rng = np.random.default_rng(1)
    x = rng.standard_normal((200, 64)) * np.exp2(rng.integers(-20, 20, (200, 1)))
    codes, k = ms.quantize_rows(x, fmt)
    xb = np.abs(x.reshape(200, 2, 32)).max(axis=-1)
    assert np.array_equal(k.astype(int), np.floor(np.log2(xb)).astype(int) - emax + 127)
    y = xb / np.exp2(k.astype(float) - 127)
    assert np.all((y >= 2.0**emax) & (y < 2.0 ** (emax + 1)))
    # a block whose max is exactly the format's largest value times a power of two is exact
    z = np.zeros((1, 32))
    z[0, 5] = ms.max_value(fmt) * 2.0**-3
    c, kk = ms.quantize_rows(z, fmt)
    assert ms.dequantize_rows(c, kk, fmt)[0, 5] == z[0, 5] and np.all(ms.dequantize_rows(c, kk, fmt)[0, :5] == 0)
    assert ms.scale_code(0.0, fmt) == 0


@pytest.mark.parametrize("fmt", list(SPEC))
def test_pack_unpack_and_bit_order(fmt):
    n = SPEC[fmt][3]
    rng = np.random.default_rng(2)
    c = rng.integers(0, n, (3, 64)).astype(np.uint8)
    p = ms.pack(c, fmt)
    assert p.shape == (3, 64 * ms.BITS[fmt] // 8)
    assert np.array_equal(ms.unpack(p, 64, fmt), c)
    if fmt == "e2m1":
        assert ms.pack(np.array([[2, 7]], np.uint8), fmt).tolist() == [[0x72]]     # element 0 in the low nibble
    else:
        # element 0 in bits 0..5, element 1 in bits 6..11, ...
        assert ms.pack(np.array([[1, 0, 0, 0]], np.uint8), fmt).tolist() == [[1, 0, 0]]
        assert ms.pack(np.array([[0, 1, 0, 0]], np.uint8), fmt).tolist() == [[0x40, 0, 0]]
        assert ms.pack(np.array([[0, 0, 0, 63]], np.uint8), fmt).tolist() == [[0, 0, 0xFC]]


# ---------------------------------------------------------------- Q and K in MXFP6 / MXFP4 inside attention
def _grid_qk(L, D, seed):
    """Q or K whose every 32-element block holds values from {1, 1.5, 2, 3, 4, 6} (signed, with
    zeros) times one power of two, and reaches 6 times that power: exactly representable in E2M3,
    E3M2, E2M1 and E4M3 under each format's own scale rule, with no subnormal element."""
    rng = np.random.default_rng(seed)
    vals = np.array([0.0, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    x = rng.choice(vals, size=(L, D)) * rng.choice([-1.0, 1.0], size=(L, D))
    x[:, ::32] = 6.0
    return x * np.exp2(rng.integers(-3, 4, size=(L, D // 32))).repeat(32, axis=1)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2", "e2m1"])
def test_attention_qk_formats_agree_on_representable_operands(fmt):
    from oracle import attention as at
    L, D = 80, 64
    q, k = _grid_qk(L, D, 1), _grid_qk(L, D, 2)
    v = np.random.default_rng(3).standard_normal((L, D))
    a = at.forward_head(q, k, v, 0.125, True, qk_fmt=fmt)
    b = at.forward_head(q, k, v, 0.125, True)
    assert np.array_equal(a["S"], b["S"]) and np.array_equal(a["O"], b["O"]) and np.array_equal(a["LSE"], b["LSE"])


def _e2m1_brute(x):
    """E2M1 quantization by search: per 32-block scale 2^(floor(log2 amax) - 2), each element the
    nearest of the eight magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} (ties to the even code), sign kept,
    6 above the top."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    out = np.zeros_like(x)
    for r in range(x.shape[0]):
        for b0 in range(0, x.shape[1], 32):
            blk = x[r, b0:b0 + 32]
            amax = np.max(np.abs(blk))
            if amax == 0:
                continue
            s = 2.0 ** (math.floor(math.log2(amax)) - 2)
            for i, y in enumerate(blk):
                d = np.abs(np.abs(y) / s - mags)
                best = np.flatnonzero(d == d.min())
                code = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
                out[r, b0 + i] = math.copysign(mags[code] * s, y)
    return out


def test_attention_e2m1_logits_match_a_brute_force_quantizer():
    from oracle import attention as at
    rng = np.random.default_rng(4)
    L, D = 40, 64
    q, k, v = (rng.standard_normal((L, D)) * 3 for _ in range(3))
    S = at.forward_head(q, k, v, 0.125, False, qk_fmt="e2m1")["S"]
    ref = (_e2m1_brute(q) @ _e2m1_brute(k).T).astype(np.float32).astype(np.float64)
    assert np.array_equal(S, ref)


@pytest.mark.parametrize("fmt,floor", [("e2m3", 0.99), ("e3m2", 0.99), ("e2m1", 0.97)])
def test_attention_qk_formats_stay_close_to_float64_attention(fmt, floor):
    from oracle import attention as at
    rng = np.random.default_rng(5)
    L, D = 96, 64
    q, k, v = (rng.standard_normal((L, D)) for _ in range(3))
    ref = at.forward_head(q, k, v, 0.125, True, quantize=False, exact=True)["O"]
    o = at.forward_head(q, k, v, 0.125, True, qk_fmt=fmt)["O"]
    assert np.sum(o * ref) / np.linalg.norm(o) / np.linalg.norm(ref) >= floor


# ---------------------------------------------------------------- square blocks (backward)
def _e2m1_brute_sq(x):
    """E2M1 square [32 x 32] blocks by search: per block scale 2^(floor(log2 amax) - 2) over all
    1024 entries, each element the nearest magnitude (ties to the even code)."""
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    out = np.zeros_like(x)
    for r0 in range(0, x.shape[0], 32):
        for c0 in range(0, x.shape[1], 32):
            blk = x[r0:r0 + 32, c0:c0 + 32]
            amax = np.max(np.abs(blk))
            if amax == 0:
                continue
            s = 2.0 ** (math.floor(math.log2(amax)) - 2)
            for (i, j), y in np.ndenumerate(blk):
                d = np.abs(np.abs(y) / s - mags)
                best = np.flatnonzero(d == d.min())
                code = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
                out[r0 + i, c0 + j] = math.copysign(mags[code] * s, y)
    return out


def test_square_blocks_e2m1_match_a_brute_force_quantizer():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((70, 64)) * np.exp2(rng.integers(-4, 5, size=(70, 1)))   # a ragged tail
    c, k = ms.quantize_sq32(x, "e2m1")
    assert np.array_equal(ms.dequantize_sq32(c, k, "e2m1"), _e2m1_brute_sq(x))


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2", "e2m1"])
def test_square_blocks_transpose_invariant_and_exact_on_representable_blocks(fmt):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((64, 64))
    c, k = ms.quantize_sq32(x, fmt)
    ct, kt = ms.quantize_sq32(x.T, fmt)
    assert np.array_equal(ct, c.T) and np.array_equal(kt, k.T)
    # values already on the grid of one block scale come back unchanged
    y = ms.dequantize_sq32(c, k, fmt)
    c2, k2 = ms.quantize_sq32(y, fmt)
    assert np.array_equal(ms.dequantize_sq32(c2, k2, fmt), y)
    # the block max sets the scale: floor(log2 amax) - emax + 127
    blk = np.abs(x[:32, :32]).max()
    assert int(k[0, 0]) == math.floor(math.log2(blk)) - ms.FORMATS[fmt][3] + 127


@pytest.mark.parametrize("fmt", ["e2m3", "e2m1"])
def test_column_packed_copy_holds_each_token_block_of_each_feature(fmt):
    rng = np.random.default_rng(8)
    x = rng.standard_normal((45, 64))              # second block row: 13 tokens, the rest zero codes
    c, _ = ms.quantize_sq32(x, fmt)
    cols = ms.pack_sq32_columns(c, fmt)
    assert cols.shape == (2, 64, 32 * ms.BITS[fmt] // 8)
    back = ms.unpack(cols, 32, fmt)                 # [2, 64, 32 tokens]
    for b in range(2):
        for f in (0, 17, 63):
            want = np.zeros(32, dtype=np.uint8)
            n = min(32, 45 - 32 * b)
            want[:n] = c[32 * b:32 * b + n, f]
            assert np.array_equal(back[b, f], want)


@pytest.mark.parametrize("fmt", ["e2m3", "e3m2", "e2m1"])
def test_backward_qk_formats_agree_on_representable_operands(fmt):
    """Q and K on a grid every square block represents exactly in the small format (and in E4M3):
    the backward in that format equals the MXFP8 backward bit for bit."""
    from oracle import attention as at
    L, D = 80, 64
    rng = np.random.default_rng(9)
    mags = np.array([1.0, 1.5, 2.0, 3.0])        # in every format's grid under a common block scale
    q = rng.choice(mags, (L, D)) * rng.choice([-1.0, 1.0], (L, D)) * 0.5
    k = rng.choice(mags, (L, D)) * rng.choice([-1.0, 1.0], (L, D)) * 0.25
    v, do = (rng.standard_normal((L, D)) for _ in range(2))
    f = at.forward_head(q, k, v, 0.125, True)
    o, lse = at.bf16(f["O"]), at.fl32(f["LSE"])
    a = at.backward_head(q, k, v, o, do, lse, 0.125, True, qk_fmt=fmt)
    b = at.backward_head(q, k, v, o, do, lse, 0.125, True)
    for n in ("dQ", "dK", "dV", "S"):
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("fmt", ["e2m3", "e2m1"])
def test_backward_qk_format_bounds_collapse_and_contain_the_oracle(fmt):
    from oracle import attention as at
    rng = np.random.default_rng(10)
    L, D = 96, 64
    q, k, v, do = (rng.standard_normal((L, D)) for _ in range(4))
    f = at.forward_head(q, k, v, 0.125, True)
    o, lse = at.bf16(f["O"]), at.fl32(f["LSE"])
    g = at.backward_head(q, k, v, o, do, lse, 0.125, True, qk_fmt=fmt)
    tight = at.backward_bounds(q, k, v, o, do, lse, 0.125, True, mma=False, fp32=False, qk_fmt=fmt)
    wide = at.backward_bounds(q, k, v, o, do, lse, 0.125, True, qk_fmt=fmt)
    for n in ("dQ", "dK", "dV"):
        scale = np.max(np.abs(g[n]))
        assert np.max(np.abs(tight[n][0] - g[n])) <= 1e-12 * scale, n
        assert np.all((wide[n][0] <= g[n]) & (g[n] <= wide[n][1])), n


@pytest.mark.parametrize("fmt,floor", [("e2m3", 0.98), ("e2m1", 0.9)])
def test_backward_qk_formats_stay_close_to_float64_gradients(fmt, floor):
    from oracle import attention as at
    rng = np.random.default_rng(11)
    L, D = 96, 64
    q, k, v, do = (rng.standard_normal((L, D)) for _ in range(4))
    ref = at.attention_fp64_backward(q, k, v, do, 0.125, True)
    f = at.forward_head(q, k, v, 0.125, True)
    g = at.backward_head(q, k, v, at.bf16(f["O"]), do, at.fl32(f["LSE"]), 0.125, True, qk_fmt=fmt)
    for i, n in enumerate(("dQ", "dK", "dV")):
        x, y = g[n], ref[i]
        assert np.sum(x * y) / np.linalg.norm(x) / np.linalg.norm(y) >= floor, n
