"""GPU parity: the fused MXFP8 attention forward against the oracle.

The oracle computes the plain definition (every product the exact sum, rounded once to fp32).
The matrix unit's products may differ from it by up to the stated bound (oracle/gemm.py), which
can move P codes, so O is several-valued: O (fp32 output) must lie within 1e-3 * max|O| of the
oracle's admissible interval, bf16 O within that plus half a bf16 ulp, LSE within 1e-4 +
1e-6 |LSE| of its interval.  Where the interval is one value this is the plain check; each test
logs how many rows needed the widening.  The grid workload makes every S product exact on the
matrix unit, so there O meets the plain bar against the exact oracle with no widening."""
import math

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx
import synth
from oracle import attention as at

from mxtest import check_lse, check_lse_bounds, check_out, check_out_bounds, log

pytestmark = pytest.mark.gpu
ALL = mx.ROW32 | mx.COL32 | mx.SQ32


def _gpu_fwd(q, k, v, sigma, causal, out_dtype):
    qq = mx.quantize(q, mx.ROW32)[mx.ROW32]
    kq = mx.quantize(k, mx.ROW32)[mx.ROW32]
    vq = mx.quantize(v, mx.COL32)[mx.COL32]
    o, lse = mx.attn_fwd(qq, kq, vq, sigma, causal, out_dtype)
    torch.cuda.synchronize()
    return o, lse


def _compare_full(q, k, v, sigma, causal, what):
    B, S, H, D = q.shape
    o32, lse = _gpu_fwd(q.cuda(), k.cuda(), v.cuda(), sigma, causal, torch.float32)
    o16, _ = _gpu_fwd(q.cuda(), k.cuda(), v.cuda(), sigma, causal, torch.bfloat16)
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    O, LSE = at.mx_attention_forward(qn, kn, vn, sigma, causal)
    lo, hi, llo, lhi = at.mx_attention_forward_bounds(qn, kn, vn, sigma, causal)
    check_out_bounds(o32.double().cpu().numpy(), lo, hi, O, f"{what} fp32-out")
    check_out_bounds(o16.double().cpu().numpy(), lo, hi, O, f"{what} bf16-out", bf16=True)
    check_lse_bounds(lse.cpu().numpy(), llo, lhi, what)


def test_forward_tiny_noncausal_fp32():
    w = synth.workload("tiny")
    log("fwd tiny")
    q, k, v = (synth.tensor_np(w, t) for t in ("q", "k", "v"))
    _compare_full(q, k, v, 1 / math.sqrt(w.D), w.causal, "tiny")


def test_forward_small_causal_outliers():
    w = synth.workload("small")
    log("fwd small")
    q, k, v = (synth.tensor_np(w, t) for t in ("q", "k", "v"))
    _compare_full(q, k, v, 1 / math.sqrt(w.D), w.causal, "small")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,H,D", [(1, 1, 1, 64), (2, 33, 2, 128), (1, 200, 3, 64), (1, 300, 2, 128)])
def test_forward_ragged_shapes(B, S, H, D, causal):
    g = torch.Generator().manual_seed(S * 7 + D)
    q, k, v = (torch.randn(B, S, H, D, generator=g).to(torch.bfloat16) for _ in range(3))
    log(f"fwd ragged {B, S, H, D} causal={causal}")
    _compare_full(q, k, v, 1 / math.sqrt(D), causal, f"ragged {(B, S, H, D)}")


def test_forward_one_hot_rows_follow_the_integer_frame():
    """Rows dominated by a single key: O equals (MX(p)/p) v-hat of that key."""
    B, S, H, D = 1, 64, 1, 64
    g = torch.Generator().manual_seed(5)
    q = (0.01 * torch.randn(B, S, H, D, generator=g))
    k = (0.01 * torch.randn(B, S, H, D, generator=g))
    v = torch.randn(B, S, H, D, generator=g)
    k[0, 7, 0, :] = 1.0
    q[0, 40:, 0, :] = 40.0
    _compare_full(q, k, v, 1.0, True, "one-hot")


def test_forward_llm_shape_sampled():
    """The metric shape (B8 H32 S8192 D128, causal, bf16 O) in the launch bench.py times; the
    seeded sample of 4 (batch, head) pairs, each on its first 40 rows, 300 random rows and the last
    row, against the oracle's admissible interval."""
    w = synth.workload("llm")
    sigma = 1 / math.sqrt(w.D)
    pairs = synth.draw_sample_pairs(w.seed, w.B, w.H, 4)
    log(f"fwd llm {w.shape()} pairs {pairs}")
    q, k, v = (synth.tensor_torch(w, t, "cuda") for t in ("q", "k", "v"))
    o, lse = _gpu_fwd(q, k, v, sigma, True, torch.bfloat16)
    rng = np.random.default_rng(0)
    for b, h in pairs:
        qs, ks, vs = (synth.head_slice_np(w, t, b, h).double().numpy() for t in ("q", "k", "v"))
        rows = np.sort(np.concatenate([np.arange(0, 40), rng.choice(w.S, 300, replace=False), [w.S - 1]]))
        rows = np.unique(rows)
        r = at.forward_head(qs, ks, vs, sigma, True, q_rows=rows)
        bd = at.forward_head_bounds(qs, ks, vs, sigma, True, q_rows=rows)
        check_out_bounds(o[b, rows, h, :].double().cpu().numpy(), bd["O_lo"], bd["O_hi"], r["O"], f"llm b{b} h{h}",
                         bf16=True)
        check_lse_bounds(lse[b, h, rows].cpu().numpy(), bd["LSE_lo"], bd["LSE_hi"], f"llm b{b} h{h}")


def test_forward_varlen_sampled():
    w = synth.workload("varlen")
    sigma = 1 / math.sqrt(w.D)
    cu = w.cu_seqlens()
    log(f"fwd varlen T={cu[-1]}")
    x = {t: synth.tensor_torch(w, t, "cuda") for t in ("q", "k", "v")}
    cu_d = torch.from_numpy(cu).cuda()
    qq, csr = mx.quantize_varlen(x["q"], cu_d, w.seqlens, mx.ROW32)
    kq, _ = mx.quantize_varlen(x["k"], cu_d, w.seqlens, mx.ROW32)
    vq, _ = mx.quantize_varlen(x["v"], cu_d, w.seqlens, mx.COL32)
    o, lse = mx.attn_fwd_varlen(qq[mx.ROW32], kq[mx.ROW32], vq[mx.COL32], cu_d, csr, w.seqlens, sigma, True,
                                torch.float32)
    torch.cuda.synchronize()
    xn = {t: x[t].double().cpu().numpy() for t in x}
    rng = np.random.default_rng(1)
    for s in range(len(w.seqlens)):
        h = int(rng.integers(w.H))
        a, b = cu[s], cu[s + 1]
        rows = np.unique(np.concatenate([np.arange(min(40, b - a)), rng.choice(b - a, 64, replace=False)]))
        args = (xn["q"][a:b, h], xn["k"][a:b, h], xn["v"][a:b, h], sigma, True)
        r = at.forward_head(*args, q_rows=rows)
        bd = at.forward_head_bounds(*args, q_rows=rows)
        check_out_bounds(o[a:b, h][rows].double().cpu().numpy(), bd["O_lo"], bd["O_hi"], r["O"], f"varlen seq{s} h{h}")
        check_lse_bounds(lse[h, a:b][rows].cpu().numpy(), bd["LSE_lo"], bd["LSE_hi"], f"varlen seq{s} h{h}")


def test_forward_is_deterministic():
    w = synth.workload("small")
    q, k, v = (synth.tensor_np(w, t).cuda() for t in ("q", "k", "v"))
    o1, l1 = _gpu_fwd(q, k, v, 0.088, True, torch.bfloat16)
    o2, l2 = _gpu_fwd(q, k, v, 0.088, True, torch.bfloat16)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("seqlens", [[1, 31, 32, 33, 200], [0, 33, 0, 200, 1, 0]])
def test_forward_varlen_short_and_empty_sequences(seqlens):
    """Jagged layout with tail blocks of every size, one-token and empty sequences (first, middle
    and last): every O row and LSE entry against the oracle."""
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    H, D = 3, 64
    sigma = 1 / math.sqrt(D)
    g = torch.Generator().manual_seed(21)
    q, k, v = (torch.randn(int(cu[-1]), H, D, generator=g).to(torch.bfloat16) for _ in range(3))
    log(f"fwd varlen {seqlens}")
    cu_d = torch.from_numpy(cu).cuda()
    qq, csr = mx.quantize_varlen(q.cuda(), cu_d, seqlens, mx.ROW32)
    kq, _ = mx.quantize_varlen(k.cuda(), cu_d, seqlens, mx.ROW32)
    vq, _ = mx.quantize_varlen(v.cuda(), cu_d, seqlens, mx.COL32)
    o, lse = mx.attn_fwd_varlen(qq[mx.ROW32], kq[mx.ROW32], vq[mx.COL32], cu_d, csr, seqlens, sigma, True,
                                torch.float32)
    torch.cuda.synchronize()
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    O, LSE = at.mx_attention_forward(qn, kn, vn, sigma, True, cu_seqlens=cu)
    lo, hi, llo, lhi = at.mx_attention_forward_bounds(qn, kn, vn, sigma, True, cu_seqlens=cu)
    check_out_bounds(o.double().cpu().numpy(), lo, hi, O, f"varlen {seqlens}")
    check_lse_bounds(lse.cpu().numpy(), llo, lhi, f"varlen {seqlens}")


def test_forward_grid_workload_meets_the_plain_bar():
    """Values +-(1 + m/8): every block scale is equal and every product of two elements lies in two
    adjacent binades, so S = Q^K^T is exact on the matrix unit and P's codes are unique.  O must
    then match the exact oracle within 1e-3 max|O| (bf16 O: plus half a bf16 ulp) and LSE within
    1e-4 + 1e-6 |LSE|, with no widening.  B2 H4 S1000 D128 causal: several query and key tiles and
    a ragged tail (1000 = 7 x 128 + 104)."""
    w = synth.workload("grid")
    sigma = 1 / math.sqrt(w.D)
    log(f"fwd grid {w.shape()}")
    q, k, v = (synth.tensor_np(w, t) for t in ("q", "k", "v"))
    o32, lse = _gpu_fwd(q.cuda(), k.cuda(), v.cuda(), sigma, True, torch.float32)
    o16, _ = _gpu_fwd(q.cuda(), k.cuda(), v.cuda(), sigma, True, torch.bfloat16)
    O, LSE = at.mx_attention_forward(*(t.double().numpy() for t in (q, k, v)), sigma, True)
    check_out(o32.double().cpu().numpy(), O, "grid fp32-out")
    check_out(o16.double().cpu().numpy(), O, "grid bf16-out", bf16=True)
    check_lse(lse.cpu().numpy(), LSE, "grid")
