"""Pins for the oracle's MX codec and quantizers (CPU only).

Each test checks the oracle against something other than itself: the OCP
anchor table, torch's own float8_e4m3fn conversion, a brute-force nearest
search, closed forms of the scale rule, and invariants of MX quantization.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _finite_codes():
    return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_decode_matches_golden_anchors():
    for line in open(os.path.join(GOLDEN, "ocp_e4m3_anchors.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = mx.e4m3_decode(np.array([int(code, 16)]))[0]
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_decode_matches_torch_float8_e4m3fn():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = mx.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])


def test_encode_decode_roundtrip_all_finite_codes():
    c = _finite_codes()
    assert np.array_equal(mx.e4m3_encode(mx.e4m3_decode(c)), c)


def _brute_encode(y):
    """Nearest finite E4M3 value; ties to the even code; saturate at 448."""
    codes = np.arange(0, 0x7F, dtype=np.int64)              # non-negative finite codes
    vals = mx.e4m3_decode(codes)
    assert np.all(np.diff(vals) > 0)
    out = []
    for x in np.asarray(y, np.float64):
        a = min(abs(x), 448.0)
        d = np.abs(vals - a)
        best = np.flatnonzero(d == d.min())
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out.append(int(c) | (0x80 if math.copysign(1.0, x) < 0 else 0))
    return np.array(out, dtype=np.uint8)


def test_encode_matches_brute_force_on_bf16_grid():
    # every bf16 bit pattern with a finite value, scaled into and around E4M3's range
    bits = np.arange(0, 1 << 16, dtype=np.uint32)
    x32 = (bits << 16).view(np.float32)
    x = x32[np.isfinite(x32)].astype(np.float64)
    rng = np.random.default_rng(7)
    for scale_exp in (0, -8, 8, 127 - 119):
        y = x * 2.0 ** scale_exp
        y = y[(np.abs(y) < 2000) & (np.abs(y) > 2.0 ** -12)]
        y = rng.choice(y, size=min(len(y), 3000), replace=False)
        assert np.array_equal(mx.e4m3_encode(y), _brute_encode(y))


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(1)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-1, 1, 20000) * 2.0 ** -6,
                        mx.e4m3_decode(_finite_codes()) * 1.0])
    # midpoints between neighbours (ties) -- exactly representable in float32
    v = mx.e4m3_decode(np.arange(0, 0x7E))
    mids = (v[:-1] + v[1:]) / 2
    y = np.concatenate([y, mids, -mids]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mx.e4m3_encode(y.astype(np.float64)), ref)


def test_encode_saturates():
    y = np.array([448.0, 460.0, 464.0, 464.01, 479.0, 480.0, 1e6, -1e30, np.inf, -np.inf])
    assert [int(c) for c in mx.e4m3_encode(y)] == [0x7E] * 7 + [0xFE, 0x7E, 0xFE]


def test_scale_rule_closed_forms():
    cases = {1.0: 119, 448.0: 127, 256.0: 127, 511.999: 127, 512.0: 128, 3 * 2.0 ** 100: 220,
             2.0 ** -130: 0, 0.0: 0, 2.0 ** -119: 0, 2.0 ** -118: 1, 0.75: 118, 2.0 ** 127 * 1.5: 246}
    got = mx.scale_code(np.array(list(cases)))
    assert [int(g) for g in got] == list(cases.values())


def test_scale_rule_against_exact_integer_log2():
    rng = np.random.default_rng(3)
    a = np.abs(rng.standard_normal(5000)) * 2.0 ** rng.integers(-100, 100, 5000)
    for x, k in zip(a, mx.scale_code(a)):
        m, e = math.frexp(x)                 # x = m 2^e, m in [0.5, 1)
        assert int(k) == min(max(e - 1 - 8 + 127, 0), 254)


def test_block_roundtrip_exact_for_representable_blocks():
    rng = np.random.default_rng(4)
    codes = rng.choice(_finite_codes(), size=(200, 32))
    codes[:, 0] = rng.choice(np.arange(0x78, 0x7F), size=200) | rng.choice([0, 0x80], 200)  # max in [256, 448]
    k = rng.integers(10, 240, size=200)
    x = mx.e4m3_decode(codes) * np.exp2(k - 127.0)[:, None]
    c2, k2 = mx.quantize_blocks(x)
    assert np.array_equal(k2, k)
    assert np.array_equal(mx.dequantize_blocks(c2, k2), x)


def test_block_saturation_artefact_of_floor_rule():
    # amax with mantissa 1.875 is beyond what the chosen scale can hold: it lands on 1.75 of its binade
    for E in (-20, 0, 13):
        x = np.zeros(32)
        x[3] = 240.0 * 2.0 ** E
        x[5] = -1.0 * 2.0 ** E
        c, k = mx.quantize_blocks(x)
        xh = mx.dequantize_blocks(c, k)
        assert xh[3] == 224.0 * 2.0 ** E and xh[5] == x[5]


def test_equivariance_under_power_of_two_scaling():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 32)) * 3
    c0, k0 = mx.quantize_blocks(x)
    for kk in (-40, -3, 1, 17):
        c1, k1 = mx.quantize_blocks(x * 2.0 ** kk)
        assert np.array_equal(c0, c1) and np.array_equal(k1.astype(int), k0.astype(int) + kk)


def test_row32_layout_and_shape_match_pages():
    facts = {}
    for line in open(os.path.join(GOLDEN, "pages_mx_facts.txt")):
        if line.strip() and not line.startswith("#"):
            key, *vals = line.split()
            facts[key] = [int(v) for v in vals]
    assert facts["block_elements"] == [mx.BLOCK] and facts["e8m0_bias"] == [mx.E8M0_BIAS]
    B, S, H, D = facts["example_qkv_shape"]
    x = np.random.default_rng(0).standard_normal((1, 64, 2, D))
    c, k = mx.quantize_row32(x)
    assert k.shape == (1, 64, 2, D // 32)
    assert list(facts["example_scale_shape"]) == [B, S, H, D // 32]
    # scales apply to 32 contiguous features
    for j in range(D // 32):
        cj, kj = mx.quantize_blocks(x[..., 32 * j:32 * j + 32])
        assert np.array_equal(cj, c[..., 32 * j:32 * j + 32]) and np.array_equal(kj, k[..., j])


def test_sq32_transpose_invariance():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((96, 128)) * np.exp(rng.standard_normal((96, 1)))
    c, k = mx.quantize_sq32(x, 0)
    ct, kt = mx.quantize_sq32(x.T.copy(), 0)
    assert np.array_equal(c, ct.T) and np.array_equal(k, kt.T)


def test_sq32_ragged_tail():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((70, 64))
    c, k = mx.quantize_sq32(x, 0)
    assert k.shape == (3, 2) and c.shape == x.shape
    blk = x[64:70, 32:64]                          # the short tail block: 6 rows x 32
    kk = mx.scale_code(np.abs(blk).max())
    assert k[2, 1] == kk
    assert np.array_equal(c[64:70, 32:64], mx.e4m3_encode(blk * 2.0 ** (127 - int(kk))))


def test_col32_equals_row32_of_transpose():
    rng = np.random.default_rng(9)
    v = rng.standard_normal((2, 96, 3, 64))
    c, k = mx.quantize_col32(v, axis=1)
    vt = np.swapaxes(v, 1, 3)                     # [2, 64, 3, 96]
    ct, kt = mx.quantize_row32(vt)
    assert np.array_equal(c, np.swapaxes(ct, 1, 3)) and np.array_equal(k, np.swapaxes(kt, 1, 3))


def test_varlen_sequences_match_fixed_length_and_pads_are_zero():
    rng = np.random.default_rng(10)
    L = [5, 128, 33, 200, 0, 64]
    cu = np.concatenate([[0], np.cumsum(L)])
    x = rng.standard_normal((cu[-1], 2, 64))
    out = mx.quantize_varlen(x, cu)
    po = mx.padded_offsets(L)
    assert np.all(po % 128 == 0)
    for s, n in enumerate(L):
        if n == 0:
            continue
        xs = x[cu[s]:cu[s + 1]]
        c, k = mx.quantize_row32(xs)
        assert np.array_equal(out["row32"][0][cu[s]:cu[s + 1]], c)
        assert np.array_equal(out["row32"][1][po[s]:po[s] + n], k)
        assert not out["row32"][1][po[s] + n:po[s + 1]].any()
        c, k = mx.quantize_col32(xs, axis=0)
        assert np.array_equal(out["col32"][0][cu[s]:cu[s + 1]], c)
        nb = k.shape[0]
        assert np.array_equal(out["col32"][1][po[s] // 32:po[s] // 32 + nb], k)
        assert not out["col32"][1][po[s] // 32 + nb:po[s + 1] // 32].any()
        c, k = mx.quantize_sq32(xs, 0)
        assert np.array_equal(out["sq32"][0][cu[s]:cu[s + 1]], c)
        assert np.array_equal(out["sq32"][1][po[s] // 32:po[s] // 32 + nb], k)
