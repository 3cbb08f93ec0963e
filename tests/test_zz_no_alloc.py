"""GPU: mx_attn_bwd_noalloc (the backward for callers that cannot allocate; its scratch is a static
device array of the library) against mx_attn_bwd with a caller workspace, on two calls in a row,
the second smaller -- so stale accumulator or flag contents from the first call would show.
dK and dV come from the same kernels in a fixed order: bitwise equal.  dQ is reduced by fp16
atomics whose order varies: within 5e-3 relative Frobenius error (the backward's bar) and within
the fp16 accumulation's spread elementwise.  The fp16 range flag must agree."""
import ctypes
import math

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx

from mxtest import log, rel_fro

pytestmark = pytest.mark.gpu


def _inputs(B, S, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    q, k, v, do = (torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).cuda() for _ in range(4))
    qs = mx.quantize(q, mx.SQ32)[mx.SQ32]
    ks = mx.quantize(k, mx.SQ32)[mx.SQ32]
    dos = mx.quantize(do, mx.SQ32)[mx.SQ32]
    vr = mx.quantize(v, mx.ROW32)[mx.ROW32]
    qq = mx.quantize(q, mx.ROW32)[mx.ROW32]
    kq = mx.quantize(k, mx.ROW32)[mx.ROW32]
    vq = mx.quantize(v, mx.COL32)[mx.COL32]
    o, lse = mx.attn_fwd(qq, kq, vq, 1 / math.sqrt(D), True, torch.bfloat16)
    return qs, ks, vr, dos, o, do, lse


def _noalloc(qs, ks, vr, dos, o, do, lse, sigma, s):
    B, S, H, D = qs[0].shape
    dq, dk, dv = (torch.empty((B, S, H, D), dtype=torch.float32, device="cuda") for _ in range(3))
    mx.mx_attn_bwd_noalloc(qs[0], qs[1], ks[0], ks[1], vr[0], vr[1], dos[0], dos[1], o, do, lse, B, S, H, D, sigma,
                           True, s, dq, dk, dv)
    return dq, dk, dv, mx.mx_attn_bwd_overflow(None)


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_backward_matches_the_workspace_backward(order):
    for (B, S, H, D, seed, s) in ((2, 1000, 4, 128, 1, 8), (1, 300, 2, 64, 2, 8)):
        log(f"noalloc bwd {(B, S, H, D)}")
        ins = _inputs(B, S, H, D, seed)
        sigma = 1 / math.sqrt(D)
        a = _noalloc(*ins, sigma, s)
        b = mx.attn_bwd(*ins[:4], ins[4], ins[5], ins[6], sigma, True, s, torch.float32, with_overflow=True)
        torch.cuda.synchronize()
        assert a[3] == b[3]
        assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
        e = rel_fro(a[0].double().cpu().numpy(), b[0].double().cpu().numpy())
        spread = float((a[0] - b[0]).abs().max() / b[0].abs().max())
        log(f"  dQ rel Frobenius {e:.2e}, max elementwise {spread:.2e} of max|dQ|")
        assert e <= 5e-3 and spread <= 2.0 ** -8


def test_noalloc_backward_raises_the_flag_like_the_workspace_backward():
    """A static scale far too large for the dQ values (2^15): both paths raise the range flag."""
    ins = _inputs(1, 256, 2, 128, 3)
    sigma = 1 / math.sqrt(128)
    a = _noalloc(*ins, sigma, 15)
    b = mx.attn_bwd(*ins[:4], ins[4], ins[5], ins[6], sigma, True, 15, torch.float32, with_overflow=True)
    assert a[3] and b[3]
    a = _noalloc(*ins, sigma, 0)
    assert not a[3]


def test_noalloc_rejects_calls_beyond_its_scratch():
    ins = _inputs(1, 64, 1, 128, 4)
    with pytest.raises(mx.MXError, match="MX_EWORKSPACE"):
        B, S, H, D = 4, 8192, 16, 128
        fake = ctypes.c_void_p(16)
        st = mx.lib().mx_attn_bwd_noalloc(*([fake] * 8), fake, fake, mx.BF16, fake, B, S, H, D, 0.1, 1, 8, fake,
                                          fake, fake, mx.F32, None)
        mx._check(st, "mx_attn_bwd_noalloc")
