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


@pytest.mark.timeout(600)
def test_backward_fmt_llm_shape_sampled_blocks():
    """MXFP4 (E2M1) Q and K at the metric shape (B8 H32 S8192 D128, causal): two seeded (batch, head)
    pairs carry O and LSE from the oracle forward (Q, K in the same format); the other heads an inert
    filler (O = 0, LSE = 30).  dQ of sampled query blocks and dK, dV of sampled key blocks against the
    oracle's block-subset gradients and admissible intervals."""
    import synth

    w = synth.workload("llm")
    B, S, H, D = w.B, w.S, w.H, w.D
    sigma = 1 / math.sqrt(D)
    pairs = synth.draw_sample_pairs(w.seed, B, H, 2)
    log(f"bwd e2m1 llm {w.shape()} heads {pairs}")
    o = torch.zeros(B, S, H, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, S), 30.0, device="cuda")
    heads = {}
    for b, h in pairs:
        qn, kn, vn, dn = (synth.head_slice_np(w, t, b, h).double().numpy() for t in ("q", "k", "v", "do"))
        on = np.zeros((S, D))
        ln = np.zeros(S)
        for r0 in range(0, S, 1024):       # the oracle forward in row chunks (every step is row-wise)
            rows = np.arange(r0, min(S, r0 + 1024))
            f = at.forward_head(qn, kn, vn, sigma, True, q_rows=rows, qk_fmt="e2m1")
            on[rows], ln[rows] = at.bf16(f["O"]), at.fl32(f["LSE"])
        o[b, :, h, :] = torch.from_numpy(on.astype(np.float32)).to(torch.bfloat16).cuda()
        lse[b, h, :] = torch.from_numpy(ln.astype(np.float32)).cuda()
        heads[(b, h)] = (qn, kn, vn, on, dn, ln)
    x = {t: synth.tensor_torch(w, t, "cuda") for t in ("q", "k", "v", "do")}
    qf, kf = mx.quantize_sq_fmt(x["q"], mx.E2M1), mx.quantize_sq_fmt(x["k"], mx.E2M1)
    vr = mx.quantize(x["v"], mx.ROW32)[mx.ROW32]
    dos = mx.quantize(x["do"], mx.SQ32)[mx.SQ32]
    dq, dk, dv = mx.attn_bwd_fmt(qf, kf, vr, dos, o, x["do"], lse, sigma, True, 8, mx.E2M1, torch.float32)
    torch.cuda.synchronize()
    del qf, kf, vr, dos, x
    rng = np.random.default_rng(12)
    nb = S // 32
    for (b, h), (qn, kn, vn, on, dn, ln) in heads.items():
        gq, gk, gv = (t[b, :, h, :].double().cpu().numpy() for t in (dq, dk, dv))
        qb = sorted({0, nb - 1, *rng.choice(nb, 2, replace=False).tolist()})
        kb = sorted({0, nb - 1, *rng.choice(nb, 2, replace=False).tolist()})
        args = (qn, kn, vn, on, dn, ln, sigma, True)
        ex = at.backward_head_blocks(*args, q_blocks=qb, k_blocks=kb, qk_fmt="e2m1")
        bd = at.backward_bounds(*args, q_blocks=qb, k_blocks=kb, qk_fmt="e2m1")
        for name, g_, bl in (("dQ", gq, qb), ("dK", gk, kb), ("dV", gv, kb)):
            rows = np.concatenate([np.arange(32 * i, min(S, 32 * i + 32)) for i in bl])
            check_grad_bounds(g_[rows], *bd[name], np.concatenate([ex[name][i] for i in bl]),
                              f"e2m1 llm b{b} h{h} {name} blocks {bl}")
