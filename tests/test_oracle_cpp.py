"""The plain C++ statement of the CPU oracle (oracle/cpp/mx_oracle.cpp), CPU only.

Pinned two ways: against what the pages and mathematics fix (the OCP E4M3 anchor table, torch's own
float8_e4m3fn conversion, a closed form of uniform attention, brute-force nearest-value encoding)
and against the NumPy oracle, value for value: bit-identical codes and scales, and attention
results equal up to the order of double-precision sums.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention as at
from oracle import mx
from tests import oracle_cpp as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_decode_matches_golden_anchors_and_torch():
    L = oc.lib()
    for line in open(os.path.join(GOLDEN, "ocp_e4m3_anchors.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        got = L.mxo_e4m3_value(int(code, 16))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([L.mxo_e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok]) and np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def _encode_grid():
    """Every finite E4M3 value, the midpoints between neighbours (ties), points just either side of
    them, values past saturation, signed zeros, infinities and a log-uniform spread."""
    vals = np.array([mx.e4m3_decode(np.array([c]))[0] for c in range(0x7F)], np.float64)   # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    rng = np.random.default_rng(5)
    spread = np.exp2(rng.uniform(-14, 10, 4000)) * rng.choice([-1.0, 1.0], 4000)
    pos = np.concatenate([vals, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf),
                          [448.0, 464.0, np.nextafter(464.0, 0), 480.0, 1e30, np.inf, 2.0 ** -10, 2.0 ** -11]])
    return np.concatenate([pos, -pos, [0.0, -0.0], spread])


def test_encode_matches_numpy_oracle_and_brute_force():
    L = oc.lib()
    y = _encode_grid()
    got = np.array([L.mxo_e4m3_code(float(v)) for v in y], np.uint8)
    assert np.array_equal(got, mx.e4m3_encode(y))
    # brute force: the nearest finite E4M3 value (ties to the even code), saturating
    codes = np.array([c for c in range(0x7F)], np.uint8)
    cand = mx.e4m3_decode(codes)
    for v, c in zip(y[np.isfinite(y)][::7], got[np.isfinite(y)][::7]):
        a = min(abs(v), 448.0)
        dist = np.abs(cand - a)
        best = codes[dist == dist.min()]
        want = best[0] if len(best) == 1 else best[(best & 1) == 0][0]
        assert (c & 0x7F) == want, (v, c, want)


def test_scale_code_closed_forms():
    L = oc.lib()
    for e in range(-140, 140):
        for f in (1.0, 1.5, np.nextafter(2.0, 0)):
            a = math.ldexp(f, e)
            assert L.mxo_scale_code(a) == min(max(e - 8 + 127, 0), 254)
    assert L.mxo_scale_code(0.0) == 0 and L.mxo_scale_code(448.0) == 127


def _blocky(rng, n, d):
    """Values whose 32-wide blocks span scales 2^-30 .. 2^30 (some blocks all zero)."""
    x = rng.standard_normal((n, d)) * np.exp2(rng.integers(-30, 31, size=(n, 1)))
    x[rng.random((n, d)) < 0.02] = 0.0
    x[:, :min(d, 32)][rng.random(n) < 0.1] = 0.0
    return x


@pytest.mark.parametrize("n,d", [(1, 32), (77, 96), (64, 128), (33, 70)])
def test_quantizers_bit_identical_to_numpy_oracle(n, d):
    rng = np.random.default_rng(n * 1000 + d)
    x = _blocky(rng, n, d)
    if d % 32 == 0:
        c, k = oc.quantize("row32", x)
        cn, kn = mx.quantize_row32(x)
        assert np.array_equal(c, cn) and np.array_equal(k, kn)
    c, k = oc.quantize("col32", x)
    cn, kn = mx.quantize_col32(x, axis=0)
    assert np.array_equal(c, cn) and np.array_equal(k, kn)
    c, k = oc.quantize("sq32", x)
    cn, kn = mx.quantize_sq32(x, 0)
    assert np.array_equal(c, cn) and np.array_equal(k, kn)


def _bf16(rng, *shape, scale=1.0):
    return torch.from_numpy(rng.standard_normal(shape) * scale).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("L,D,causal", [(1, 64, True), (45, 64, False), (100, 128, True), (70, 128, False)])
def test_forward_matches_numpy_oracle(L, D, causal):
    rng = np.random.default_rng(L + D)
    q, k, v = _bf16(rng, L, D, scale=2.0), _bf16(rng, L, D, scale=2.0), _bf16(rng, L, D)
    sigma = 1 / math.sqrt(D)
    O, lse, pc, ps = oc.attn_fwd(q, k, v, sigma, causal)
    ref = at.forward_head(q, k, v, sigma, causal)
    vis = at.visible(L, L, causal)
    assert np.array_equal(np.where(vis, pc, 0), np.where(vis, ref["P_codes"], 0))
    assert np.array_equal(ps, ref["P_scales"])
    assert np.allclose(O, ref["O"], rtol=1e-12, atol=1e-12 * np.max(np.abs(ref["O"])))
    assert np.allclose(lse, ref["LSE"], rtol=1e-12, atol=1e-12)


def test_forward_uniform_attention_closed_form():
    """q = 0: every visible logit is 0, so M = 0, p = 1 exactly, every P code is 1.0 under scale
    2^-8, and O_i is the mean of the visible rows of V-hat, LSE_i = ln(number of visible keys)."""
    rng = np.random.default_rng(3)
    L, D = 67, 64
    v = _bf16(rng, L, D)
    O, lse, pc, ps = oc.attn_fwd(np.zeros((L, D)), _bf16(rng, L, D), v, 0.125, True)
    vc, vk = mx.quantize_col32(v, axis=0)
    vh = mx.dequantize_col32(vc, vk, axis=0)
    for i in range(L):
        assert np.allclose(O[i], vh[:i + 1].mean(axis=0), rtol=1e-13, atol=1e-15)
        assert lse[i] == pytest.approx(math.log(i + 1), rel=1e-14)
        assert np.all(pc[i, :i + 1] == 0x78) and np.all(ps[i, :(i + 32) // 32] == 119)


@pytest.mark.parametrize("L,D,causal", [(40, 64, True), (96, 128, False), (75, 128, True)])
def test_backward_matches_numpy_oracle(L, D, causal):
    rng = np.random.default_rng(10 * L + D)
    q, k, v, do = (_bf16(rng, L, D) for _ in range(4))
    sigma = 1 / math.sqrt(D)
    f = at.forward_head(q, k, v, sigma, causal)
    o = torch.from_numpy(f["O"]).to(torch.bfloat16).double().numpy()
    lse = f["LSE"].astype(np.float32).astype(np.float64)
    dq, dk, dv, Dv = oc.attn_bwd(q, k, v, o, do, lse, sigma, causal)
    ref = at.backward_head(q, k, v, o, do, lse, sigma, causal)
    assert np.array_equal(Dv, ref["D"])
    for got, want in ((dq, ref["dQ"]), (dk, ref["dK"]), (dv, ref["dV"])):
        assert np.allclose(got, want, rtol=1e-11, atol=1e-12 * np.max(np.abs(want)))
