"""GPU parity: the fused attention backward with Q and K in MXFP6 / MXFP4 (mx_attn_bwd_fmt) against
the oracle's backward in the same formats.

Q and K are quantized in square [32 x 32] blocks in the small element format (row-packed for
S = Q^ K^T, column-packed for dK = dS^T Q^ and dQ = dS^ K^); dO and V stay MXFP8, and P and dS are
quantized online in MXFP8.  Both sides receive the same bytes (Q, K, V, dO from a seeded generator;
O and LSE from the oracle forward with Q, K in the same format).  The bar is test_gpu_bwd's: per
head, the part of each gradient outside the oracle's admissible interval (backward_bounds with the
format) stays within 5e-3 relative Frobenius error of the exact gradient."""
import math

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx
from oracle import attention as at

from mxtest import check_grad_bounds, log

pytestmark = pytest.mark.gpu
FMTS = {mx.E2M3: "e2m3", mx.E3M2: "e3m2", mx.E2M1: "e2m1"}


def _fwd_inputs(q, k, v, sigma, causal, name, cu=None):
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    O, LSE = at.mx_attention_forward(qn, kn, vn, sigma, causal, cu_seqlens=cu, qk_fmt=name)
    return torch.from_numpy(O.astype(np.float32)).to(torch.bfloat16), torch.from_numpy(LSE.astype(np.float32))


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,S,H", [(1, 1, 1), (2, 100, 2), (1, 300, 1)])
def test_backward_fmt_ragged_shapes(fmt, causal, B, S, H):
    D = 128
    name = FMTS[fmt]
    g = torch.Generator().manual_seed(S + fmt)
    q, k, v, do = (torch.randn(B, S, H, D, generator=g).to(torch.bfloat16) for _ in range(4))
    sigma = 1 / math.sqrt(D)
    log(f"bwd {name} {(B, S, H, D)} causal={causal}")
    o, lse = _fwd_inputs(q, k, v, sigma, causal, name)
    dev = "cuda"
    qf, kf = mx.quantize_sq_fmt(q.to(dev), fmt), mx.quantize_sq_fmt(k.to(dev), fmt)
    vr = mx.quantize(v.to(dev), mx.ROW32)[mx.ROW32]
    dos = mx.quantize(do.to(dev), mx.SQ32)[mx.SQ32]
    qn, kn, vn, on, don = (t.double().numpy() for t in (q, k, v, o, do))
    ln = lse.double().numpy()
    for gd in (torch.float32, torch.bfloat16):
        out = mx.attn_bwd_fmt(qf, kf, vr, dos, o.to(dev), do.to(dev), lse.to(dev), sigma, causal, 8, fmt, gd,
                              with_overflow=True)
        torch.cuda.synchronize()
        assert not out[3]
        gpu = [t.double().cpu().numpy() for t in out[:3]]
        for b in range(B):
            for h in range(H):
                args = (qn[b, :, h], kn[b, :, h], vn[b, :, h], on[b, :, h], don[b, :, h], ln[b, h], sigma, causal)
                ex = at.backward_head(*args, qk_fmt=name)
                bd = at.backward_bounds(*args, qk_fmt=name)
                for i, n in enumerate(("dQ", "dK", "dV")):
                    check_grad_bounds(gpu[i][b, :, h], *bd[n], ex[n], f"{name} b{b} h{h} {n} {gd}")


@pytest.mark.parametrize("fmt", [mx.E2M3, mx.E2M1])
def test_backward_fmt_varlen(fmt):
    """Jagged layout with empty and one-token sequences; every (sequence, head) against the oracle."""
    name = FMTS[fmt]
    seqlens = [5, 130, 0, 77, 1, 200]
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    H, D = 2, 128
    sigma = 1 / math.sqrt(D)
    g = torch.Generator().manual_seed(7 + fmt)
    q, k, v, do = (torch.randn(int(cu[-1]), H, D, generator=g).to(torch.bfloat16) for _ in range(4))
    log(f"bwd {name} varlen T={cu[-1]}")
    o, lse = _fwd_inputs(q, k, v, sigma, True, name, cu)
    dev = "cuda"
    cu_d = torch.from_numpy(cu).to(dev)
    csr = torch.empty(len(seqlens) + 1, dtype=torch.int32, device=dev)
    mx.mx_varlen_scale_offsets(cu_d, len(seqlens), csr)
    qf = mx.quantize_sq_fmt_varlen(q.to(dev), cu_d, csr, seqlens, fmt)
    kf = mx.quantize_sq_fmt_varlen(k.to(dev), cu_d, csr, seqlens, fmt)
    dos, _ = mx.quantize_varlen(do.to(dev), cu_d, seqlens, mx.SQ32)
    vr, _ = mx.quantize_varlen(v.to(dev), cu_d, seqlens, mx.ROW32)
    out = mx.attn_bwd_fmt_varlen(qf, kf, vr[mx.ROW32], dos[mx.SQ32], o.to(dev), do.to(dev), lse.to(dev), cu_d, csr,
                                 seqlens, sigma, True, 8, fmt, torch.float32)
    torch.cuda.synchronize()
    gpu = [t.double().cpu().numpy() for t in out]
    qn, kn, vn, on, don = (t.double().numpy() for t in (q, k, v, o, do))
    ln = lse.double().numpy()
    for s in range(len(seqlens)):
        a, b = cu[s], cu[s + 1]
        if a == b:
            continue
        for h in range(H):
            args = (qn[a:b, h], kn[a:b, h], vn[a:b, h], on[a:b, h], don[a:b, h], ln[h, a:b], sigma, True)
            ex = at.backward_head(*args, qk_fmt=name)
            bd = at.backward_bounds(*args, qk_fmt=name)
            for i, n in enumerate(("dQ", "dK", "dV")):
                check_grad_bounds(gpu[i][a:b, h], *bd[n], ex[n], f"{name} varlen seq{s} h{h} {n}")


def test_backward_fmt_e4m3_is_the_mxfp8_backward():
    """qk_format = E4M3 through the format entry is mx_attn_bwd: dK, dV bit for bit, dQ (summed by
    atomics in any order) to fp16 rounding."""
    B, S, H, D = 1, 150, 2, 128
    sigma = 1 / math.sqrt(D)
    g = torch.Generator().manual_seed(3)
    q, k, v, do = (torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).cuda() for _ in range(4))
    o = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).cuda()
    lse = torch.full((B, H, S), 5.0).cuda()
    qs, ks, dos = (mx.quantize(t, mx.SQ32)[mx.SQ32] for t in (q, k, do))
    vr = mx.quantize(v, mx.ROW32)[mx.ROW32]
    a = mx.attn_bwd(qs, ks, vr, dos, o, do, lse, sigma, True, 8, torch.float32)
    b = mx.attn_bwd_fmt((qs[0], None, qs[1]), (ks[0], None, ks[1]), vr, dos, o, do, lse, sigma, True, 8, mx.E4M3,
                        torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert torch.allclose(a[0], b[0], rtol=2e-3, atol=1e-6 * float(a[0].abs().max()))
