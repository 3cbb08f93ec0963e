"""GPU parity of the MX GEMM with a quantizing epilogue (mx_gemm_quantize).

The oracle's C is the exact product rounded once to fp32; the block-scaled matrix instruction
may differ from it by up to the stated bound (oracle/gemm.py, product_error_bound), so C is
several-valued and must lie within that bound of the exact sum.  C's MX codes then follow from
the C the kernel holds: the oracle quantizer applied to the kernel's own fp32 C must give every
code and scale exactly -- a complete check of the codes for whichever admissible C it computed."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx
from oracle import gemm as gm
from oracle import mx as omx

from mxtest import log, to_np

pytestmark = pytest.mark.gpu
ALL = mx.ROW32 | mx.COL32 | mx.SQ32


def _operand(rows, K, seed, spread=2.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, K)) * np.exp(rng.standard_normal((rows, 1)) * spread)
    x = x.astype(np.float32).astype(np.float64)
    codes, k = omx.quantize_row32(x)
    deq = omx.dequantize_row32(codes, k)
    expo = omx.element_exponent_row32(codes, k)
    return codes, k, deq, expo


def _run(M, N, K, seed, layouts=ALL):
    ac, ak, ad, ae = _operand(M, K, seed)
    bc, bk, bd, be = _operand(N, K, seed + 1)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.uint8)).cuda()  # noqa: E731
    out, c32 = mx.gemm_quantize((t(ac), t(ak)), (t(bc), t(bk)), layouts, with_f32=True)
    torch.cuda.synchronize()
    return out, c32.double().cpu().numpy(), (ad, ae, bd, be)


def _check_codes(out, c, what):
    # ROW32 blocks run along the columns, with a short tail block when N % 32 != 0
    ref = {mx.ROW32: omx.quantize_col32(c, axis=1), mx.COL32: omx.quantize_col32(c, axis=0),
           mx.SQ32: omx.quantize_sq32(c, 0)}
    for lay, (d, s) in out.items():
        rc, rs = ref[lay]
        gd, gs = to_np(d), to_np(s)
        assert gd.shape == rc.shape and gs.shape == rs.shape, (what, lay, gd.shape, rc.shape, gs.shape, rs.shape)
        nd, ns = int(np.sum(gd != rc)), int(np.sum(gs != rs))
        if nd:
            idx = np.argwhere(gd != rc)[:8]
            log(f"{what} {mx.LAYOUT_NAMES[lay]} mismatches at {idx.tolist()}: gpu "
                f"{[int(gd[tuple(i)]) for i in idx]} oracle {[int(rc[tuple(i)]) for i in idx]} "
                f"c {[float(c[tuple(i)]) for i in idx]}")
        assert nd == 0 and ns == 0, f"{what} {mx.LAYOUT_NAMES[lay]}: {nd} payload, {ns} scale mismatches"


def _check_c(c, ops, what, rows=None, cols=None):
    ad, ae, bd, be = ops
    if rows is not None:
        ad, ae, bd, be, c = ad[rows], ae[rows], bd[cols], be[cols], c[np.ix_(rows, cols)]
    exact = ad @ bd.T
    eps = gm.product_error_bound(gm.magnitudes(ad, ae), gm.magnitudes(bd, be))
    err = np.abs(c - exact)
    assert np.all(err <= eps), (what, float(np.max(err / np.maximum(eps, 1e-300))))
    return float(np.mean(c == gm.fl32(exact)))


@pytest.mark.parametrize("M,N,K", [(128, 128, 64), (200, 144, 192), (37, 48, 128), (256, 512, 1024),
                                   (1, 16, 64), (130, 272, 320)])
def test_gemm_quantize_exact_codes_and_admissible_c(M, N, K):
    out, c, ops = _run(M, N, K, seed=M + N + K)
    frac = _check_c(c, ops, f"{M}x{N}x{K}")
    log(f"gemm {M}x{N}x{K}: {100 * frac:.1f}% of C bit-equal to the exact product rounded once")
    _check_codes(out, c, f"{M}x{N}x{K}")


def test_gemm_quantize_single_layouts_and_f32_only():
    M, N, K = 96, 64, 128
    for lay in (mx.ROW32, mx.COL32, mx.SQ32):
        out, c, _ = _run(M, N, K, seed=5, layouts=lay)
        assert set(out) == {lay}
        _check_codes(out, c, f"layout {lay}")
    out, c, ops = _run(M, N, K, seed=5, layouts=0)
    assert out == {}
    _check_c(c, ops, "f32 only")


def test_gemm_quantize_large_sampled():
    M, N, K = 2048, 1024, 2048
    out, c, ops = _run(M, N, K, seed=11)
    rng = np.random.default_rng(3)
    rows = np.sort(rng.choice(M, 48, replace=False))
    cols = np.sort(rng.choice(N, 48, replace=False))
    _check_c(c, ops, "large sampled", rows, cols)
    for bm, bn in ((0, 0), (17, 5), (M // 32 - 1, N // 32 - 1)):
        rs, cs = slice(32 * bm, 32 * bm + 32), slice(32 * bn, 32 * bn + 32)
        blk = c[rs, cs]
        sub = {}
        for lay, (d, s) in out.items():
            d = d[rs, cs]
            s = {mx.ROW32: s[rs, bn:bn + 1], mx.COL32: s[bm:bm + 1, cs], mx.SQ32: s[bm:bm + 1, bn:bn + 1]}[lay]
            sub[lay] = (d.contiguous(), s.contiguous())
        _check_codes(sub, blk, f"large block {bm},{bn}")


def test_gemm_quantize_rejects_bad_arguments():
    a = torch.zeros(64, 64, dtype=torch.uint8, device="cuda")
    s = torch.zeros(64, 2, dtype=torch.uint8, device="cuda")
    c = torch.zeros(64, 64, dtype=torch.uint8, device="cuda")
    cs = torch.zeros(64, 2, dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MXError):   # K not a multiple of 64
        mx.mx_gemm_quantize(a, s, a, s, mx.E4M3, 64, 64, 32, mx.ROW32, c, cs, None, None, None, None, None)
    with pytest.raises(mx.MXError):   # N not a multiple of 16
        mx.mx_gemm_quantize(a, s, a, s, mx.E4M3, 64, 40, 64, mx.ROW32, c, cs, None, None, None, None, None)
    with pytest.raises(mx.MXError):   # nothing to write
        mx.mx_gemm_quantize(a, s, a, s, mx.E4M3, 64, 64, 64, 0, None, None, None, None, None, None, None)


@pytest.mark.parametrize("M,N,K", [(200, 144, 192), (130, 272, 320), (37, 48, 128), (33, 16, 64)])
def test_gemm_quantize_writes_only_its_outputs(M, N, K):
    """Every output sits between guard bands of a known byte; ragged shapes (row and column
    tiles, 32-blocks and 16-column halves past the end) must leave the bands untouched."""
    G = 512
    ac, ak, _, _ = _operand(M, K, seed=7)
    bc, bk, _, _ = _operand(N, K, seed=8)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).astype(np.uint8)).cuda()  # noqa: E731
    nbm, nbn = (M + 31) // 32, (N + 31) // 32
    sizes = [M * N, M * nbn, M * N, nbm * N, M * N, nbm * nbn]
    bufs = [torch.full((G + s + G,), 0xA5, dtype=torch.uint8, device="cuda") for s in sizes]
    views = [b[G:G + s] for b, s in zip(bufs, sizes)]
    cbuf = torch.full((G + M * N + G,), -7.0, dtype=torch.float32, device="cuda")
    mx.mx_gemm_quantize(t(ac), t(ak), t(bc), t(bk), mx.E4M3, M, N, K, ALL, *views, cbuf[G:G + M * N])
    torch.cuda.synchronize()
    for b, s in zip(bufs, sizes):
        h = to_np(b)
        assert np.all(h[:G] == 0xA5) and np.all(h[G + s:] == 0xA5), (M, N, K, s)
    hc = cbuf.cpu().numpy()
    assert np.all(hc[:G] == -7.0) and np.all(hc[G + M * N:] == -7.0)
    c = hc[G:G + M * N].reshape(M, N).astype(np.float64)
    shp = {mx.ROW32: (M, nbn), mx.COL32: (nbm, N), mx.SQ32: (nbm, nbn)}
    out = {lay: (views[2 * i].view(M, N), views[2 * i + 1].view(shp[lay]))
           for i, lay in enumerate((mx.ROW32, mx.COL32, mx.SQ32))}
    _check_codes(out, c, f"guarded {M}x{N}x{K}")
