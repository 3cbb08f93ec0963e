"""GPU parity: the fused attention forward with Q and K in MXFP6 (E2M3, E3M2) or MXFP4 (E2M1)
(mx_attn_fwd_fmt; P and V stay MXFP8) against the oracle's forward with the same Q/K element
format.  Q and K are quantized by mx_quantize_rows (bit-exact with the oracle's codec, tested in
test_gpu_mxsmall.py).  As for the MXFP8 forward, the oracle computes the plain definition and O
must lie within 1e-3 * max|O| of its admissible interval (bf16 O plus half a bf16 ulp), LSE
within 1e-4 + 1e-6 |LSE| of its interval."""
import math

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx
import synth
from oracle import attention as at

from mxtest import check_lse_bounds, check_out_bounds, log

pytestmark = pytest.mark.gpu
FMTS = {mx.E2M3: "e2m3", mx.E3M2: "e3m2", mx.E2M1: "e2m1"}


def _gpu_fwd(q, k, v, sigma, causal, fmt, out_dtype):
    B, S, H, D = q.shape
    qd = mx.quantize_rows(q.reshape(-1, D), fmt)
    kd = mx.quantize_rows(k.reshape(-1, D), fmt)
    vq = mx.quantize(v, mx.COL32)[mx.COL32]
    o, lse = mx.attn_fwd_fmt(qd, kd, vq, (B, S, H, D), sigma, causal, fmt, out_dtype)
    torch.cuda.synchronize()
    return o, lse


def _compare_full(q, k, v, sigma, causal, fmt, what):
    o32, lse = _gpu_fwd(q.cuda(), k.cuda(), v.cuda(), sigma, causal, fmt, torch.float32)
    o16, _ = _gpu_fwd(q.cuda(), k.cuda(), v.cuda(), sigma, causal, fmt, torch.bfloat16)
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    O, LSE = at.mx_attention_forward(qn, kn, vn, sigma, causal, qk_fmt=FMTS[fmt])
    lo, hi, llo, lhi = at.mx_attention_forward_bounds(qn, kn, vn, sigma, causal, qk_fmt=FMTS[fmt])
    check_out_bounds(o32.double().cpu().numpy(), lo, hi, O, f"{what} fp32-out")
    check_out_bounds(o16.double().cpu().numpy(), lo, hi, O, f"{what} bf16-out", bf16=True)
    check_lse_bounds(lse.cpu().numpy(), llo, lhi, what)


@pytest.mark.parametrize("fmt", list(FMTS))
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,H,D", [(1, 1, 1, 64), (2, 33, 2, 128), (1, 200, 3, 64), (1, 300, 2, 128)])
def test_forward_qk_format_ragged_shapes(fmt, B, S, H, D, causal):
    g = torch.Generator().manual_seed(S * 7 + D + fmt)
    q, k, v = (torch.randn(B, S, H, D, generator=g).to(torch.bfloat16) for _ in range(3))
    log(f"fwd {FMTS[fmt]} ragged {B, S, H, D} causal={causal}")
    _compare_full(q, k, v, 1 / math.sqrt(D), causal, fmt, f"{FMTS[fmt]} ragged {(B, S, H, D)}")


@pytest.mark.parametrize("fmt", list(FMTS))
def test_forward_qk_format_small_workload(fmt):
    w = synth.workload("small")
    log(f"fwd {FMTS[fmt]} small")
    q, k, v = (synth.tensor_np(w, t) for t in ("q", "k", "v"))
    _compare_full(q, k, v, 1 / math.sqrt(w.D), w.causal, fmt, f"{FMTS[fmt]} small")


def test_forward_e2m1_llm_shape_sampled():
    w = synth.workload("llm")
    sigma = 1 / math.sqrt(w.D)
    pairs = synth.draw_sample_pairs(w.seed, w.B, w.H, 1)
    log(f"fwd e2m1 llm {w.shape()} pairs {pairs}")
    q, k, v = (synth.tensor_torch(w, t, "cuda") for t in ("q", "k", "v"))
    o, lse = _gpu_fwd(q, k, v, sigma, True, mx.E2M1, torch.bfloat16)
    rng = np.random.default_rng(2)
    for b, h in pairs:
        qs, ks, vs = (synth.head_slice_np(w, t, b, h).double().numpy() for t in ("q", "k", "v"))
        rows = np.unique(np.concatenate([np.arange(0, 40), rng.choice(w.S, 200, replace=False), [w.S - 1]]))
        r = at.forward_head(qs, ks, vs, sigma, True, q_rows=rows, qk_fmt="e2m1")
        bd = at.forward_head_bounds(qs, ks, vs, sigma, True, q_rows=rows, qk_fmt="e2m1")
        check_out_bounds(o[b, rows, h, :].double().cpu().numpy(), bd["O_lo"], bd["O_hi"], r["O"], f"e2m1 llm b{b} h{h}",
                         bf16=True)
        check_lse_bounds(lse[b, h, rows].cpu().numpy(), bd["LSE_lo"], bd["LSE_hi"], f"e2m1 llm b{b} h{h}")


def test_forward_fmt_with_e4m3_is_the_mxfp8_forward():
    """qk_format MX_E4M3 with the row quantizer's output gives mx_attn_fwd's bytes exactly."""
    g = torch.Generator().manual_seed(11)
    B, S, H, D = 2, 300, 2, 128
    q, k, v = (torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).cuda() for _ in range(3))
    o1, l1 = _gpu_fwd(q, k, v, 0.088, True, mx.E4M3, torch.float32)
    qq = mx.quantize(q, mx.ROW32)[mx.ROW32]
    kq = mx.quantize(k, mx.ROW32)[mx.ROW32]
    vq = mx.quantize(v, mx.COL32)[mx.COL32]
    o2, l2 = mx.attn_fwd(qq, kq, vq, 0.088, True, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("fmt", [mx.E3M2, mx.E2M1])
def test_forward_qk_format_varlen_sampled(fmt):
    """Jagged layout: packed sequences (lengths 256..8192), Q, K scale rows at 128-aligned offsets."""
    w = synth.workload("varlen")
    sigma = 1 / math.sqrt(w.D)
    cu = w.cu_seqlens()
    log(f"fwd {FMTS[fmt]} varlen T={cu[-1]}")
    x = {t: synth.tensor_torch(w, t, "cuda") for t in ("q", "k", "v")}
    cu_d = torch.from_numpy(cu).cuda()
    vq, csr = mx.quantize_varlen(x["v"], cu_d, w.seqlens, mx.COL32)
    qf = mx.quantize_rows_varlen(x["q"], cu_d, csr, w.seqlens, fmt)
    kf = mx.quantize_rows_varlen(x["k"], cu_d, csr, w.seqlens, fmt)
    o, lse = mx.attn_fwd_fmt_varlen(qf, kf, vq[mx.COL32], cu_d, csr, w.seqlens, sigma, True, fmt, torch.float32)
    torch.cuda.synchronize()
    xn = {t: x[t].double().cpu().numpy() for t in x}
    rng = np.random.default_rng(3 + fmt)
    for s in range(len(w.seqlens)):
        h = int(rng.integers(w.H))
        a, b = cu[s], cu[s + 1]
        rows = np.unique(np.concatenate([np.arange(min(40, b - a)), rng.choice(b - a, 48, replace=False)]))
        args = (xn["q"][a:b, h], xn["k"][a:b, h], xn["v"][a:b, h], sigma, True)
        r = at.forward_head(*args, q_rows=rows, qk_fmt=FMTS[fmt])
        bd = at.forward_head_bounds(*args, q_rows=rows, qk_fmt=FMTS[fmt])
        check_out_bounds(o[a:b, h][rows].double().cpu().numpy(), bd["O_lo"], bd["O_hi"], r["O"],
                         f"{FMTS[fmt]} varlen seq{s} h{h}")
        check_lse_bounds(lse[h, a:b][rows].cpu().numpy(), bd["LSE_lo"], bd["LSE_hi"], f"{FMTS[fmt]} varlen seq{s} h{h}")
