"""GPU: gfx950's block-scaled fp8 instruction (v_mfma_scale_f32_32x32x64_f8f6f4) run alone, through
the test-only probe tests/hw/mfma_probe.hip.

  * Its result stays within the oracle's stated product bound (oracle/gemm.py) of the exact sum on
    dense random operands of wide range, sparse operands, operands with 50x outliers and a
    structured one-large-many-small case: the hardware half of the claim that the tolerance reading
    covers the matrix unit (the CPU half checks the model below against the bound).
  * On grid operands (magnitudes 1 + m/8) it equals the exact sum rounded once: the premise of the
    grid workloads, whose attention results are checked at the plain bar.
  * The measured model of its accumulation (tests/hw/mfma_model.py) reproduces it on >= 90% of the
    dot products: a characterisation of the instruction, used only by CPU tests, never as an
    expected value."""
import ctypes
import os

import numpy as np
import pytest
import torch

from hw import mfma_model
from oracle import gemm, mx

pytestmark = pytest.mark.gpu
LIB = os.path.join(os.path.dirname(__file__), "hw", "libmfmaprobe.so")


def _lanes_operand(M):
    """Logical [32 rows x 64 k] codes -> [64 lanes x 32 bytes]: lane r + 32g holds
    row r, k = 16g + j (j < 16) and 32 + 16g + (j - 16) (j >= 16)."""
    out = np.zeros((64, 32), np.uint8)
    for l in range(64):
        r, g = l % 32, l // 32
        out[l, :16] = M[r, 16 * g:16 * g + 16]
        out[l, 16:] = M[r, 32 + 16 * g:32 + 16 * g + 16]
    return out


def _lanes_scale(s):     # s [32 rows, 2 blocks]; lane r + 32b holds (r, b)
    return np.array([s[l % 32, l // 32] for l in range(64)], np.int32)


def _unlane_c(c):        # [64, 16] -> [32, 32]
    g = np.zeros((32, 32), np.float32)
    for l in range(64):
        for i in range(16):
            g[8 * (i // 4) + 4 * (l // 32) + i % 4, l % 32] = c[l, i]
    return g


def _run(cases):
    L = ctypes.CDLL(LIB)
    A = torch.from_numpy(np.stack([_lanes_operand(a) for a, _, _, _ in cases])).cuda()
    B = torch.from_numpy(np.stack([_lanes_operand(b) for _, b, _, _ in cases])).cuda()
    SA = torch.from_numpy(np.stack([_lanes_scale(s) for _, _, s, _ in cases])).cuda()
    SB = torch.from_numpy(np.stack([_lanes_scale(s) for _, _, _, s in cases])).cuda()
    out = torch.zeros(len(cases), 64, 16, dtype=torch.float32, device="cuda")
    assert L.mfma_probe(ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(B.data_ptr()), ctypes.c_void_p(SA.data_ptr()),
                        ctypes.c_void_p(SB.data_ptr()), ctypes.c_void_p(out.data_ptr()), len(cases)) == 0
    return [_unlane_c(c) for c in out.cpu().numpy()]


def _model(a, b, sa, sb):
    ka = np.repeat(sa.astype(np.int64) - 127, 32, axis=1)
    kb = np.repeat(sb.astype(np.int64) - 127, 32, axis=1)
    return mfma_model.matmul_mfma(mx.e4m3_decode(a) * np.exp2(ka), mx.e4m3_exponent(a) + ka,
                            mx.e4m3_decode(b) * np.exp2(kb), mx.e4m3_exponent(b) + kb).astype(np.float32)


def test_model_characterises_the_instruction():
    rng = np.random.default_rng(123)
    rc = lambda shape: (rng.integers(0x08, 0x7E, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)  # noqa
    cases, kinds = [], []
    unit = np.full((32, 2), 127)
    for nz in ([0, 1], list(range(8)), list(range(16)), [3, 40]):      # sparse operands
        a = np.zeros((32, 64), np.uint8)
        b = np.zeros((32, 64), np.uint8)
        a[:, nz] = rc((32, len(nz)))
        b[:, nz] = rc((32, len(nz)))
        cases.append((a, b, unit, unit)); kinds.append("sparse")
    for _ in range(4):                                                 # dense, random block scales
        cases.append((rc((32, 64)), rc((32, 64)), rng.integers(120, 135, (32, 2)), rng.integers(120, 135, (32, 2))))
        kinds.append("dense")
    a = np.full((32, 64), 0x38, np.uint8)                              # one large product beside small ones
    b = np.full((32, 64), 0x01, np.uint8)
    b[:, 0] = 0x60
    cases.append((a, b, unit, unit)); kinds.append("structured")
    got = _run(cases)
    for (a, b, sa, sb), g, kind in zip(cases, got, kinds):
        m = _model(a, b, sa, sb)
        exact = np.mean(m == g)
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(m), 1e-30))) - 23)
        worst = np.max(np.abs(m.astype(np.float64) - g) / ulp)
        print(f"{kind}: bit-exact {exact:.3f}, worst {worst:.1f} ulp", flush=True)
        if kind == "structured":
            assert exact == 1.0
        else:
            assert exact >= 0.9 and worst <= 16


def _dequant(a, s):
    k = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    return mx.e4m3_decode(a) * np.exp2(k), mx.e4m3_exponent(a) + k


def test_instruction_stays_inside_the_stated_bound():
    rng = np.random.default_rng(321)
    rc = lambda shape: (rng.integers(0x01, 0x7E, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)  # noqa
    cases = []
    for _ in range(6):                                                 # dense, wide block-scale range
        cases.append((rc((32, 64)), rc((32, 64)), rng.integers(100, 150, (32, 2)), rng.integers(100, 150, (32, 2))))
    for _ in range(4):                                                 # outliers: a few top-binade codes
        a, b = rc((32, 64)) & 0xBF, rc((32, 64)) & 0xBF                # exponents <= 7 ...
        a[rng.random(a.shape) < 0.03] = 0x7E                           # ... and some at 448
        b[rng.random(b.shape) < 0.03] = 0xFE
        cases.append((a, b, np.full((32, 2), 127), np.full((32, 2), 127)))
    for nz in ([0, 1], list(range(8)), [3, 40]):                       # sparse
        a = np.zeros((32, 64), np.uint8)
        b = np.zeros((32, 64), np.uint8)
        a[:, nz] = rc((32, len(nz)))
        b[:, nz] = rc((32, len(nz)))
        cases.append((a, b, np.full((32, 2), 127), np.full((32, 2), 127)))
    got = _run(cases)
    worst = 0.0
    for (a, b, sa, sb), g in zip(cases, got):
        av, ae = _dequant(a, sa)
        bv, be = _dequant(b, sb)
        eps = gemm.product_error_bound(gemm.magnitudes(av, ae), gemm.magnitudes(bv, be))
        err = np.abs(g.astype(np.float64) - av @ bv.T)
        worst = max(worst, float(np.max(err / np.maximum(eps, 1e-300))))
        assert np.all(err <= eps)
    print(f"largest |instruction - exact| / bound: {worst:.3f}", flush=True)


def test_grid_operands_are_added_exactly():
    rng = np.random.default_rng(5)
    grid_codes = np.array([0x38 + m for m in range(8)])                # 1 + m/8 in E4M3
    cases = []
    for _ in range(4):
        a = rng.choice(grid_codes, (32, 64)) | (rng.integers(0, 2, (32, 64)) << 7)
        b = rng.choice(grid_codes, (32, 64)) | (rng.integers(0, 2, (32, 64)) << 7)
        s = np.full((32, 2), 127 - 2)
        cases.append((a.astype(np.uint8), b.astype(np.uint8), s, s))
    for (a, b, sa, sb), g in zip(cases, _run(cases)):
        av, _ = _dequant(a, sa)
        bv, _ = _dequant(b, sb)
        assert np.array_equal(g, (av @ bv.T).astype(np.float32))
