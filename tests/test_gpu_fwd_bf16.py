"""GPU parity: the BF16 attention forward (the baseline of the MX speed-ups)
against the oracle's BF16 reading (no MX step, P rounded to bfloat16 before
P V).  Same bar as the MXFP8 forward: O within 1e-3 * max|O| (bf16 O: plus
half a bf16 ulp), LSE within 1e-4 + 1e-6 |LSE|."""
import math

import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx
import synth
from oracle import attention as at

from mxtest import check_lse, check_out, log

pytestmark = pytest.mark.gpu


def _compare_full(q, k, v, sigma, causal, what):
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    o32, lse = mx.attn_fwd_bf16(q.cuda(), k.cuda(), v.cuda(), sigma, causal, torch.float32)
    o16, _ = mx.attn_fwd_bf16(q.cuda(), k.cuda(), v.cuda(), sigma, causal, torch.bfloat16)
    torch.cuda.synchronize()
    qn, kn, vn = (t.double().numpy() for t in (q, k, v))
    O, LSE = at.mx_attention_forward(qn, kn, vn, sigma, causal, bf16_baseline=True)
    check_out(o32.double().cpu().numpy(), O, f"{what} fp32-out")
    check_out(o16.double().cpu().numpy(), O, f"{what} bf16-out", bf16=True)
    check_lse(lse.cpu().numpy(), LSE, what)


def test_bf16_forward_tiny_and_small():
    for name in ("tiny", "small"):
        w = synth.workload(name)
        log(f"bf16 fwd {name}")
        q, k, v = (synth.tensor_np(w, t) for t in ("q", "k", "v"))
        _compare_full(q, k, v, 1 / math.sqrt(w.D), w.causal, name)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,S,H,D", [(1, 1, 1, 64), (2, 33, 2, 128), (1, 200, 3, 64), (1, 300, 2, 128)])
def test_bf16_forward_ragged_shapes(B, S, H, D, causal):
    g = torch.Generator().manual_seed(S * 11 + D)
    q, k, v = (torch.randn(B, S, H, D, generator=g) for _ in range(3))
    log(f"bf16 fwd ragged {B, S, H, D} causal={causal}")
    _compare_full(q, k, v, 1 / math.sqrt(D), causal, f"ragged {(B, S, H, D)}")


def test_bf16_forward_large_logits_move_the_frame():
    """Rows whose logits grow along the keys make the lazy frame move several times."""
    B, S, H, D = 1, 256, 2, 64
    g = torch.Generator().manual_seed(9)
    q = torch.randn(B, S, H, D, generator=g)
    k = torch.randn(B, S, H, D, generator=g) * torch.linspace(0.1, 6.0, S)[None, :, None, None]
    v = torch.randn(B, S, H, D, generator=g)
    _compare_full(q, k, v, 1.0, False, "growing logits")


def test_bf16_forward_llm_shape_sampled():
    w = synth.workload("llm")
    sigma = 1 / math.sqrt(w.D)
    pairs = synth.draw_sample_pairs(w.seed, w.B, w.H, 2)
    log(f"bf16 fwd llm {w.shape()} pairs {pairs}")
    q, k, v = (synth.tensor_torch(w, t, "cuda") for t in ("q", "k", "v"))
    o, lse = mx.attn_fwd_bf16(q, k, v, sigma, True, torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    for b, h in pairs:
        qs, ks, vs = (synth.head_slice_np(w, t, b, h).double().numpy() for t in ("q", "k", "v"))
        rows = np.unique(np.concatenate([np.arange(0, 40), rng.choice(w.S, 300, replace=False), [w.S - 1]]))
        r = at.forward_head(qs, ks, vs, sigma, True, quantize=False, p_round="bf16", q_rows=rows)
        check_out(o[b, rows, h, :].double().cpu().numpy(), r["O"], f"llm b{b} h{h}", bf16=True)
        check_lse(lse[b, h, rows].cpu().numpy(), r["LSE"], f"llm b{b} h{h}")


def test_bf16_forward_varlen_sampled():
    w = synth.workload("varlen")
    sigma = 1 / math.sqrt(w.D)
    cu = w.cu_seqlens()
    log(f"bf16 fwd varlen T={cu[-1]}")
    x = {t: synth.tensor_torch(w, t, "cuda") for t in ("q", "k", "v")}
    cu_d = torch.from_numpy(cu).cuda()
    o, lse = mx.attn_fwd_bf16_varlen(x["q"], x["k"], x["v"], cu_d, w.seqlens, sigma, True, torch.float32)
    torch.cuda.synchronize()
    xn = {t: x[t].double().cpu().numpy() for t in x}
    rng = np.random.default_rng(1)
    for s in range(len(w.seqlens)):
        h = int(rng.integers(w.H))
        a, b = cu[s], cu[s + 1]
        rows = np.unique(np.concatenate([np.arange(min(40, b - a)), rng.choice(b - a, 64, replace=False)]))
        r = at.forward_head(xn["q"][a:b, h], xn["k"][a:b, h], xn["v"][a:b, h], sigma, True, quantize=False,
                            p_round="bf16", q_rows=rows)
        check_out(o[a:b, h][rows].double().cpu().numpy(), r["O"], f"varlen seq{s} h{h}")
        check_lse(lse[h, a:b][rows].cpu().numpy(), r["LSE"], f"varlen seq{s} h{h}")


def test_bf16_forward_rejects_bad_arguments():
    x = torch.zeros(1, 8, 1, 64, dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(x)
    with pytest.raises(mx.MXError):
        mx.mx_attn_fwd_bf16(x, x, x, 1, 8, 1, 96, 0.1, True, o, None)     # D
    with pytest.raises(mx.MXError):
        mx.mx_attn_fwd_bf16(x, x, x, 1, 8, 1, 64, -1.0, True, o, None)    # softmax_scale
