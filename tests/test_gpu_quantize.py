"""GPU parity: mx_quantize / mx_quantize_varlen codes and scales are
bit-exact against the oracle, on the workload shapes, ragged lengths and
adversarial blocks."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx
import synth
from oracle import mx as omx

from mxtest import assert_quant_equal, log, oracle_quant_fixed, to_np

pytestmark = pytest.mark.gpu
ALL = mx.ROW32 | mx.COL32 | mx.SQ32


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_quantize_workloads_exact(name):
    w = synth.workload(name)
    log(f"quantize {name} {w.shape()}")
    for which in ("q", "k", "v", "do"):
        x = synth.tensor_np(w, which)
        out = mx.quantize(x.cuda(), ALL)
        torch.cuda.synchronize()
        assert_quant_equal(out, oracle_quant_fixed(x.double().numpy(), ALL), f"{name}/{which}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(2, 70, 3, 64), (1, 45, 2, 128), (3, 1, 1, 128), (1, 96, 5, 64)])
def test_quantize_ragged_lengths_exact(shape, dtype):
    g = torch.Generator().manual_seed(sum(shape))
    x = (torch.randn(shape, generator=g) * torch.exp(torch.randn(shape[0], 1, shape[2], 1, generator=g) * 3)).to(dtype)
    log(f"quantize ragged {shape} {dtype}")
    for lay in (mx.ROW32, mx.COL32, mx.SQ32, ALL):
        out = mx.quantize(x.cuda(), lay)
        torch.cuda.synchronize()
        assert_quant_equal(out, oracle_quant_fixed(x.double().numpy(), lay), f"{shape}")


def _adversarial():
    """fp32 [1, 64, 2, 128]: zero blocks, subnormals, exact E4M3 ties, saturating
    maxima, -0.0, huge and tiny exponents, values at the fp32 extremes."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((1, 64, 2, 128)).astype(np.float32)
    x[0, 0:32, 0, 0:32] = 0.0                                            # all-zero square block
    x[0, 1, 1, :] = -0.0
    x[0, 2, 1, 0:32] = np.float32(1e-40) * rng.standard_normal(32).astype(np.float32)  # subnormal block
    x[0, 3, 1, 32:64] = np.float32(2.0 ** -130)
    vals = omx.e4m3_decode(np.arange(0x08, 0x7E))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)              # exact ties at scale 2^0
    x[0, 4, 1, 0:32] = mids[:32]
    x[0, 4, 1, 0] = 256.0                                                # fixes the block scale at 2^0
    x[0, 5, 1, 0:32] = -mids[32:64]
    x[0, 5, 1, 1] = -256.0
    x[0, 6, 1, 0:32] = 240.0                                             # amax mantissa 1.875: saturates
    x[0, 6, 1, 3] = 239.0
    x[0, 7, 1, 64:96] = np.float32(3.0 * 2.0 ** 100)
    x[0, 7, 1, 70] = np.float32(1.0)
    x[0, 8, 1, 96:128] = np.float32(2.0 ** 127) * 1.5
    x[0, 9, 1, 0:32] = np.float32(2.0 ** -119)
    x[0, 10, 1, 0:32] = np.float32(2.0 ** -118) * np.linspace(0.01, 1, 32).astype(np.float32)
    x[0, 40:64, 0, 64:96] = np.float32(464.0) * 2.0 ** -3                # tie to even at the top
    x[0, 41, 0, 64] = np.float32(500.0) * 2.0 ** -3
    return x


def test_quantize_adversarial_blocks_exact():
    x = _adversarial()
    for dtype in (torch.float32, torch.bfloat16):
        xt = torch.from_numpy(x).to(dtype)
        out = mx.quantize(xt.cuda(), ALL)
        torch.cuda.synchronize()
        assert_quant_equal(out, oracle_quant_fixed(xt.double().numpy(), ALL), f"adversarial {dtype}")


def test_quantize_long_context_head_scales_sampled():
    w = synth.workload("long")
    log(f"quantize long {w.shape()} (2 heads compared)")
    for which in ("q", "do"):
        x = synth.tensor_torch(w, which, "cuda")
        out = mx.quantize(x, ALL)
        torch.cuda.synchronize()
        for h in (0, 11):
            sub = {lay: (d[:, :, h:h + 1].contiguous(), s[:, :, h:h + 1].contiguous()) for lay, (d, s) in out.items()}
            xh = x[:, :, h:h + 1].double().cpu().numpy()
            assert_quant_equal(sub, oracle_quant_fixed(xh, ALL), f"long/{which}/h{h}")


def test_quantize_llm_shape_sampled_pairs():
    w = synth.workload("llm")
    pairs = synth.draw_sample_pairs(w.seed, w.B, w.H, 2)
    log(f"quantize llm {w.shape()} pairs {pairs}")
    x = synth.tensor_torch(w, "k", "cuda")
    out = mx.quantize(x, ALL)
    torch.cuda.synchronize()
    for b, h in pairs:
        xs = synth.head_slice_np(w, "k", b, h)
        assert torch.equal(xs, x[b, :, h, :].cpu()), "GPU and CPU generators disagree"
        xh = xs.double().numpy()[None, :, None, :]
        sub = {lay: (d[b:b + 1, :, h:h + 1].contiguous(), s[b:b + 1, :, h:h + 1].contiguous())
               for lay, (d, s) in out.items()}
        assert_quant_equal(sub, oracle_quant_fixed(xh, ALL), f"llm b{b} h{h}")


@pytest.mark.parametrize("seqlens", [[5, 128, 33, 200, 0, 64, 1], None])
def test_quantize_varlen_exact_and_pads_zero(seqlens):
    if seqlens is None:
        w = synth.workload("varlen")
        seqlens = w.seqlens
        x = synth.tensor_torch(w, "v", "cuda")
        heads = [0, 9]
    else:
        g = torch.Generator().manual_seed(3)
        x = torch.randn(sum(seqlens), 3, 128, generator=g).to(torch.bfloat16).cuda()
        heads = [0, 1, 2]
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    log(f"quantize varlen T={cu[-1]} nseq={len(seqlens)}")
    out, csr = mx.quantize_varlen(x, torch.from_numpy(cu).cuda(), seqlens, ALL)
    torch.cuda.synchronize()
    po = omx.padded_offsets(seqlens)
    assert np.array_equal(csr.cpu().numpy(), po)
    xn = x.double().cpu().numpy()
    for h in heads:
        ref = omx.quantize_varlen(xn[:, h:h + 1], cu)
        for lay, key in ((mx.ROW32, "row32"), (mx.COL32, "col32"), (mx.SQ32, "sq32")):
            assert np.array_equal(to_np(out[lay][0])[:, h:h + 1], ref[key][0]), (key, h)
            assert np.array_equal(to_np(out[lay][1])[:, h:h + 1], ref[key][1]), (key, h)


def test_quantize_is_deterministic():
    w = synth.workload("small")
    x = synth.tensor_np(w, "q").cuda()
    a = mx.quantize(x, ALL)
    b = mx.quantize(x, ALL)
    torch.cuda.synchronize()
    for lay in a:
        assert torch.equal(a[lay][0], b[lay][0]) and torch.equal(a[lay][1], b[lay][1])
