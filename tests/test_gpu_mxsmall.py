"""GPU parity of the MXFP6 / MXFP4 payload path: the operand quantizer
(mx_quantize_rows) must give the oracle's packed bytes and scales exactly in
every element format, and the MX GEMM must accept every format through the
matrix instruction's format fields: C within the stated product bound
(oracle/gemm.py) of the exact sum of the dequantized products, and the MXFP8
codes of C equal to the oracle quantizer applied to the kernel's own C."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx
from oracle import gemm as gm
from oracle import mx as omx
from oracle import mxsmall as ms

from mxtest import log, to_np

pytestmark = pytest.mark.gpu
FMTS = {mx.E4M3: "e4m3", mx.E2M3: "e2m3", mx.E3M2: "e3m2", mx.E2M1: "e2m1"}


def _oracle_rows(x, fmt):
    """(packed bytes, scales, dequantized values, element exponents) of x [rows, K]."""
    if fmt == mx.E4M3:
        c, k = omx.quantize_row32(x)
        return c, k, omx.dequantize_row32(c, k), omx.element_exponent_row32(c, k)
    name = FMTS[fmt]
    c, k = ms.quantize_rows(x, name)
    return ms.pack(c, name), k, ms.dequantize_rows(c, k, name), ms.element_exponent_rows(c, k, name)


def _data(rows, K, seed, spread=3.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)) * np.exp(rng.standard_normal((rows, 1)) * spread)
    x[0] = 0.0                                     # an all-zero row
    x[1, :32] = np.linspace(-7.5, 7.5, 32)         # a block holding every sixteenth-step
    x[2] = rng.standard_normal(K) * 1e-30          # tiny values (scale clamps at 0)
    x[3, ::7] = 1e4                                # large values next to small ones
    return x


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_rows_matches_the_oracle_bit_for_bit(fmt, dtype):
    rows, K = 300, 256
    xt = torch.from_numpy(_data(rows, K, 1 + fmt)).to(dtype)
    x = xt.double().numpy()
    # exact ties of the format's grid, scaled into a block whose max fixes the scale
    if fmt != mx.E4M3:
        name = FMTS[fmt]
        v = ms.decode(np.arange(2 ** (ms.BITS[name] - 1)), name)
        mids = (v[1:] + v[:-1]) / 2
        row = np.zeros(K)
        row[0] = ms.max_value(name)
        row[1:1 + len(mids[:31])] = mids[:31]
        x[5] = row
        xt = torch.from_numpy(x).to(dtype)
        x = xt.double().numpy()
    d, s = mx.quantize_rows(xt.cuda(), fmt)
    torch.cuda.synchronize()
    rd, rs, _, _ = _oracle_rows(x, fmt)
    gd, gs = to_np(d), to_np(s)
    assert gd.shape == rd.shape and gs.shape == rs.shape
    nd, ns = int(np.sum(gd != rd)), int(np.sum(gs != rs))
    if nd:
        idx = np.argwhere(gd != rd)[:6]
        log(f"{FMTS[fmt]} mismatches at {idx.tolist()}: gpu {[int(gd[tuple(i)]) for i in idx]} "
            f"oracle {[int(rd[tuple(i)]) for i in idx]}")
    assert nd == 0 and ns == 0, f"{FMTS[fmt]} {dtype}: {nd} byte and {ns} scale mismatches"


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("M,N,K", [(200, 144, 192), (128, 256, 512), (37, 48, 64)])
def test_gemm_in_every_element_format(fmt, M, N, K):
    a = _data(M, K, 10 + fmt, spread=2.0)
    b = _data(N, K, 20 + fmt, spread=2.0)
    ad, ak, av, ae = _oracle_rows(a, fmt)
    bd, bk, bv, be = _oracle_rows(b, fmt)
    t = lambda z: torch.from_numpy(np.ascontiguousarray(z).astype(np.uint8)).cuda()  # noqa: E731
    out, c = mx.gemm_quantize((t(ad), t(ak)), (t(bd), t(bk)), mx.ROW32 | mx.COL32 | mx.SQ32, with_f32=True,
                              fmt=fmt)
    torch.cuda.synchronize()
    c = c.double().cpu().numpy()
    exact = av @ bv.T
    bound = gm.product_error_bound(gm.magnitudes(av, ae), gm.magnitudes(bv, be))
    assert np.all(np.abs(c - exact) <= bound), (FMTS[fmt], float(np.max(np.abs(c - exact) / bound)))
    log(f"gemm {FMTS[fmt]} {M}x{N}x{K}: {100 * float(np.mean(c == exact.astype(np.float32))):.1f}% of C "
        f"bit-equal to fl32(exact)")
    ref = {mx.ROW32: omx.quantize_col32(c, axis=1), mx.COL32: omx.quantize_col32(c, axis=0),
           mx.SQ32: omx.quantize_sq32(c, 0)}
    for lay, (dd, ss) in out.items():
        assert np.array_equal(to_np(dd), ref[lay][0]) and np.array_equal(to_np(ss), ref[lay][1]), (FMTS[fmt], lay)


def test_gemm_from_the_gpu_quantizer_end_to_end():
    """Operands produced by mx_quantize_rows (bf16 input) feed the GEMM directly."""
    M, N, K = 256, 128, 1024
    g = torch.Generator().manual_seed(3)
    a = torch.randn(M, K, generator=g).to(torch.bfloat16)
    b = torch.randn(N, K, generator=g).to(torch.bfloat16)
    for fmt in FMTS:
        qa, qb = mx.quantize_rows(a.cuda(), fmt), mx.quantize_rows(b.cuda(), fmt)
        _, c = mx.gemm_quantize(qa, qb, 0, with_f32=True, fmt=fmt)
        torch.cuda.synchronize()
        _, _, av, _ = _oracle_rows(a.double().numpy(), fmt)
        _, _, bv, _ = _oracle_rows(b.double().numpy(), fmt)
        exact = av @ bv.T
        bound = 2.0 ** -8 * (np.abs(av) @ np.abs(bv).T) + 1e-30
        err = np.abs(c.double().cpu().numpy() - exact)
        assert np.all(err <= bound), FMTS[fmt]
        # the quantized product approximates the bf16 product (looser for fewer bits)
        full = a.double().numpy() @ b.double().numpy().T
        rel = float(np.linalg.norm(c.double().cpu().numpy() - full) / np.linalg.norm(full))
        log(f"end to end {FMTS[fmt]}: rel Frobenius error vs the unquantized product {rel:.3e}")
        assert rel < {mx.E4M3: 0.05, mx.E2M3: 0.1, mx.E3M2: 0.2, mx.E2M1: 0.4}[fmt]


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("seqlens", [[5, 128, 33, 200, 0, 64], [0, 1, 0, 300, 0]])
def test_quantize_rows_varlen_places_scale_rows_at_the_padded_offsets(fmt, seqlens):
    """mx_quantize_rows_varlen: payload rows at the packed token positions, scale rows at the
    oracle's 128-aligned per-sequence offsets (empty sequences own none), pad rows 0, every byte
    equal to the oracle's per-sequence row quantization."""
    H, D = 3, 64
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    T = int(cu[-1])
    x = _data(T * H, D, 40 + fmt).reshape(T, H, D)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    x = xt.double().numpy()
    cu_d = torch.from_numpy(cu).cuda()
    csr = torch.empty(len(seqlens) + 1, dtype=torch.int32, device="cuda")
    mx.mx_varlen_scale_offsets(cu_d, len(seqlens), csr)
    d, s = mx.quantize_rows_varlen(xt.cuda(), cu_d, csr, seqlens, fmt)
    torch.cuda.synchronize()
    po = omx.padded_offsets(seqlens)
    assert to_np(csr).tolist() == po.tolist()
    gd, gs = to_np(d), to_np(s)
    ref_s = np.zeros_like(gs)
    for i in range(len(seqlens)):
        a, b = cu[i], cu[i + 1]
        if a == b:
            continue
        rd, rs, _, _ = _oracle_rows(x[a:b].reshape(-1, D), fmt)
        assert np.array_equal(gd[a:b].reshape(rd.shape), rd), (FMTS[fmt], i)
        ref_s[po[i]:po[i] + (b - a)] = rs.reshape(b - a, H, D // 32)
    assert np.array_equal(gs, ref_s), FMTS[fmt]


SMALL = [mx.E2M3, mx.E3M2, mx.E2M1]


def _oracle_sq(xh, fmt):
    """Row-packed bytes [L, D w/8], column-packed bytes [ceil(L/32), D, 32 w/8], scales of one head."""
    name = FMTS[fmt]
    c, k = ms.quantize_sq32(xh, name)
    return ms.pack(c, name), ms.pack_sq32_columns(c, name), k


@pytest.mark.parametrize("fmt", SMALL)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(2, 70, 3, 128), (1, 33, 2, 64)])
def test_quantize_sq_fmt_matches_the_oracle_bit_for_bit(fmt, dtype, shape):
    """mx_quantize_sq_fmt: square blocks in a small format, row-packed and column-packed payloads and
    the scales equal to the oracle's, byte for byte (ragged tails, mixed magnitudes, zero blocks)."""
    B, S, H, D = shape
    x = _data(B * S * H, D, 60 + fmt).reshape(B, S, H, D)
    x[0, 32:64, 0, :32] = 0.0                       # one all-zero square block
    xt = torch.from_numpy(x).to(dtype)
    x = xt.double().numpy()
    row, col, sc = mx.quantize_sq_fmt(xt.cuda(), fmt)
    torch.cuda.synchronize()
    gr, gc, gs = to_np(row), to_np(col), to_np(sc)
    for b in range(B):
        for h in range(H):
            rr, rc, rk = _oracle_sq(x[b, :, h, :], fmt)
            assert np.array_equal(gr[b, :, h], rr), (FMTS[fmt], b, h, "row")
            assert np.array_equal(gc[b, :, h], rc), (FMTS[fmt], b, h, "col")
            assert np.array_equal(gs[b, :, h], rk), (FMTS[fmt], b, h, "scale")


@pytest.mark.parametrize("fmt", SMALL)
def test_quantize_sq_fmt_varlen_places_block_rows_at_the_padded_offsets(fmt):
    """mx_quantize_sq_fmt_varlen: row-packed payload at the packed token positions; column-packed
    blocks and scales at the 128-aligned per-sequence block rows; pad block rows all zero."""
    seqlens = [5, 128, 0, 70, 200]
    H, D = 2, 128
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    T = int(cu[-1])
    x = _data(T * H, D, 80 + fmt).reshape(T, H, D)
    xt = torch.from_numpy(x).to(torch.bfloat16)
    x = xt.double().numpy()
    cu_d = torch.from_numpy(cu).cuda()
    csr = torch.empty(len(seqlens) + 1, dtype=torch.int32, device="cuda")
    mx.mx_varlen_scale_offsets(cu_d, len(seqlens), csr)
    row, col, sc = mx.quantize_sq_fmt_varlen(xt.cuda(), cu_d, csr, seqlens, fmt)
    torch.cuda.synchronize()
    po = omx.padded_offsets(seqlens)
    gr, gc, gs = to_np(row), to_np(col), to_np(sc)
    ref_c, ref_s = np.zeros_like(gc), np.zeros_like(gs)
    for i in range(len(seqlens)):
        a, b = cu[i], cu[i + 1]
        if a == b:
            continue
        nb = (b - a + 31) // 32
        for h in range(H):
            rr, rc, rk = _oracle_sq(x[a:b, h, :], fmt)
            assert np.array_equal(gr[a:b, h], rr), (FMTS[fmt], i, h)
            ref_c[po[i] // 32:po[i] // 32 + nb, h] = rc
            ref_s[po[i] // 32:po[i] // 32 + nb, h] = rk
    assert np.array_equal(gc, ref_c) and np.array_equal(gs, ref_s), FMTS[fmt]
