"""GPU parity: the BF16 attention backward (the baseline of the MX backward)
against the oracle's BF16 reading (no MX step; P and dS rounded to bfloat16
before their products).  Both sides receive the same bytes: Q, K, V, dO
(bf16), O (bf16) and LSE (fp32) from the oracle's BF16 forward.  dQ, dK, dV
must match within 5e-3 relative Frobenius error per tensor, the bar of the
MXFP8 backward; the kernels add no atomics, so every output is bitwise
repeatable."""
import math

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx
import synth
from oracle import attention as at

from mxtest import log, rel_fro

pytestmark = pytest.mark.gpu
TOL = 5e-3


def _inputs(B, S, H, D, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.randn(B, S, H, D, generator=g).to(torch.bfloat16) for _ in range(4)]


def _oracle_fwd(q, k, v, sigma, causal, cu=None):
    O, LSE = at.mx_attention_forward(*(t.double().numpy() for t in (q, k, v)), sigma, causal, cu_seqlens=cu,
                                     bf16_baseline=True)
    return torch.from_numpy(O.astype(np.float32)).to(torch.bfloat16), torch.from_numpy(LSE.astype(np.float32))


def _check(gpu, ref, what):
    for name, a, b in zip(("dQ", "dK", "dV"), gpu, ref):
        # a single visible key per query makes dS (so dQ, dK) exactly zero: then compare absolutely
        e = rel_fro(a, b) if np.any(b != 0) else float(np.max(np.abs(a)))
        log(f"  {what} {name}: rel Frobenius {e:.2e}")
        assert np.all(np.isfinite(a)), f"{what} {name}: non-finite values"
        assert e <= TOL, f"{what} {name}: rel Frobenius {e:.3e} > {TOL}"


def _run(q, k, v, do, sigma, causal, grad_dtype):
    o, lse = _oracle_fwd(q, k, v, sigma, causal)
    d = lambda t: t.cuda()  # noqa: E731
    out = mx.attn_bwd_bf16(d(q), d(k), d(v), d(o), d(do), d(lse), sigma, causal, grad_dtype)
    torch.cuda.synchronize()
    ref = at.mx_attention_backward(*(t.double().numpy() for t in (q, k, v, o, do)), lse.double().numpy(), sigma,
                                   causal, bf16_baseline=True)
    return [t.double().cpu().numpy() for t in out], ref


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("B,S,H,D", [(1, 1, 1, 64), (1, 200, 2, 64), (2, 100, 3, 128), (1, 300, 1, 128),
                                     (1, 129, 2, 128)])
def test_bf16_backward_ragged_shapes(B, S, H, D, causal):
    q, k, v, do = _inputs(B, S, H, D, S + 3 * D)
    log(f"bf16 bwd ragged {(B, S, H, D)} causal={causal}")
    for gd in (torch.float32, torch.bfloat16):
        gpu, ref = _run(q, k, v, do, 1 / math.sqrt(D), causal, gd)
        _check(gpu, ref, f"ragged {(B, S, H, D)} {gd}")


def test_bf16_backward_many_tiles():
    """1100 queries: several 128-key workgroups and 64-query steps, a ragged last tile."""
    q, k, v, do = _inputs(1, 1100, 2, 128, 7)
    log("bf16 bwd 1100 tokens")
    gpu, ref = _run(q, k, v, do, 1 / math.sqrt(128), True, torch.float32)
    _check(gpu, ref, "1100 causal")


def test_bf16_backward_small_workload_outliers():
    w = synth.workload("small")
    q, k, v, do = (synth.tensor_np(w, t)[:, :, :4] for t in ("q", "k", "v", "do"))
    q, k, v, do = (t.contiguous() for t in (q, k, v, do))
    log("bf16 bwd small (4 heads)")
    gpu, ref = _run(q, k, v, do, 1 / math.sqrt(w.D), True, torch.float32)
    _check(gpu, ref, "small")


def test_bf16_backward_varlen():
    seqlens = [5, 130, 300, 77, 1, 64]
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    H, D = 2, 128
    sigma = 1 / math.sqrt(D)
    g = torch.Generator().manual_seed(99)
    q, k, v, do = (torch.randn(int(cu[-1]), H, D, generator=g).to(torch.bfloat16) for _ in range(4))
    log(f"bf16 bwd varlen T={cu[-1]}")
    o, lse = _oracle_fwd(q, k, v, sigma, True, cu)
    cu_d = torch.from_numpy(cu).cuda()
    gpu = mx.attn_bwd_bf16_varlen(q.cuda(), k.cuda(), v.cuda(), o.cuda(), do.cuda(), lse.cuda(), cu_d, seqlens,
                                  sigma, True, torch.float32)
    torch.cuda.synchronize()
    ref = at.mx_attention_backward(*(t.double().numpy() for t in (q, k, v, o, do)), lse.double().numpy(), sigma,
                                   True, cu_seqlens=cu, bf16_baseline=True)
    _check([t.double().cpu().numpy() for t in gpu], ref, "varlen")


def test_bf16_backward_is_bitwise_repeatable():
    q, k, v, do = (t.cuda() for t in _inputs(2, 512, 4, 128, 5))
    o, lse = mx.attn_fwd_bf16(q, k, v, 1 / math.sqrt(128), True, torch.bfloat16)
    a = mx.attn_bwd_bf16(q, k, v, o, do, lse, 1 / math.sqrt(128), True, torch.float32)
    b = mx.attn_bwd_bf16(q, k, v, o, do, lse, 1 / math.sqrt(128), True, torch.float32)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.isfinite(x).all() and torch.equal(x, y)


def test_bf16_backward_rejects_bad_arguments():
    x = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(1, 1, 8, device="cuda")
    ws = torch.empty(mx.mx_attn_bwd_bf16_workspace_bytes(8, 1), dtype=torch.uint8, device="cuda")
    with pytest.raises(mx.MXError):   # workspace too small
        mx.mx_attn_bwd_bf16(x, x, x, x, x, lse, 1, 8, 1, 64, 0.1, True, x, x, x, ws[:16])
    with pytest.raises(mx.MXError):   # D
        mx.mx_attn_bwd_bf16(x, x, x, x, x, lse, 1, 8, 1, 80, 0.1, True, x, x, x, ws)


def test_bf16_backward_llm_shape_sampled_head():
    """The metric shape (B8 H32 S8192 D128, causal, bf16 gradients) in the call bench.py times.
    One sampled (batch, head) carries O and LSE from the oracle's BF16 forward; every other head
    holds an inert filler (O = 0, LSE = 30, so its p is ~0).  The sampled head's whole dQ, dK and
    dV are compared with the oracle's BF16 backward."""
    w = synth.workload("llm")
    B, S, H, D = w.B, w.S, w.H, w.D
    sigma = 1 / math.sqrt(D)
    (b, h), = synth.draw_sample_pairs(w.seed + 1, B, H, 1)
    log(f"bf16 bwd llm {w.shape()} head {(b, h)}")
    x = {t: synth.tensor_torch(w, t, "cuda") for t in ("q", "k", "v", "do")}
    qn, kn, vn, dn = (synth.head_slice_np(w, t, b, h).double().numpy() for t in ("q", "k", "v", "do"))
    f = at.forward_head(qn, kn, vn, sigma, True, quantize=False, p_round="bf16")
    o_h = torch.from_numpy(f["O"].astype(np.float32)).to(torch.bfloat16)
    lse_h = torch.from_numpy(f["LSE"].astype(np.float32))
    del f
    o = torch.zeros(B, S, H, D, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, S), 30.0, device="cuda")
    o[b, :, h, :] = o_h.cuda()
    lse[b, h, :] = lse_h.cuda()
    dq, dk, dv = mx.attn_bwd_bf16(x["q"], x["k"], x["v"], o, x["do"], lse, sigma, True, torch.bfloat16)
    torch.cuda.synchronize()
    gpu = [t[b, :, h, :].double().cpu().numpy() for t in (dq, dk, dv)]
    del dq, dk, dv, x, o, lse
    r = at.backward_head(qn, kn, vn, o_h.double().numpy(), dn, lse_h.double().numpy(), sigma, True,
                         quantize=False, p_round="bf16")
    _check(gpu, (r["dQ"], r["dK"], r["dV"]), f"llm b{b} h{h}")
