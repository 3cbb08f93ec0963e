"""GPU parity: mx_rmsnorm_quantize / mx_rmsnorm_quantize_varlen codes and
scales are bit-exact against the oracle (RMSNorm over D per (token, head),
then the quantizer), on ragged shapes, adversarial rows, the jagged layout
and sampled blocks of the metric shape."""
import numpy as np
import pytest
import torch

import mxfp8_block_scaled_flash_amd as mx
import synth
from oracle import mx as omx
from oracle import norm as onorm

from mxtest import assert_quant_equal, log, oracle_quant_fixed, to_np

pytestmark = pytest.mark.gpu
ALL = mx.ROW32 | mx.COL32 | mx.SQ32


def _gamma(D, seed):
    g = torch.Generator().manual_seed(seed)
    return (1 + 0.25 * torch.randn(D, generator=g)).float()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(2, 70, 3, 128), (1, 45, 2, 64), (3, 1, 1, 128), (1, 96, 5, 64)])
def test_rmsnorm_quantize_ragged_exact(shape, dtype):
    g = torch.Generator().manual_seed(100 + sum(shape))
    x = (torch.randn(shape, generator=g) * torch.exp(torch.randn(shape[0], 1, shape[2], 1, generator=g) * 3)).to(dtype)
    gamma = _gamma(shape[-1], sum(shape))
    eps = 1e-6
    log(f"rmsnorm quantize {shape} {dtype}")
    y = onorm.rmsnorm(x.double().numpy(), gamma.double().numpy(), eps)
    for lay in (mx.ROW32, ALL):
        out = mx.rmsnorm_quantize(x.cuda(), gamma.cuda(), eps, lay)
        torch.cuda.synchronize()
        assert_quant_equal(out, oracle_quant_fixed(y, lay), f"{shape} {dtype}")


def test_rmsnorm_quantize_adversarial_rows():
    """Zero rows (eps only), a single dominant element, tiny and huge rows, negative gains."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((1, 64, 2, 128)).astype(np.float32)
    x[0, 0, 0, :] = 0.0
    x[0, 1, 0, :] = 0.0
    x[0, 1, 0, 17] = 3.0e4
    x[0, 2, 1, :] *= np.float32(2.0 ** -60)
    x[0, 3, 1, :] *= np.float32(2.0 ** 60)
    x[0, 4:36, 1, :] = 1.0                      # a whole constant block: y = gamma
    gamma = rng.standard_normal(128).astype(np.float32)
    gamma[5] = 0.0
    for eps in (0.0, 1e-5):
        for dtype in (torch.float32, torch.bfloat16):
            xt = torch.from_numpy(x).to(dtype)
            if eps == 0.0:
                xt[0, 0, 0, :] = 1.0            # no all-zero row without eps
            y = onorm.rmsnorm(xt.double().numpy(), gamma.astype(np.float64), eps)
            out = mx.rmsnorm_quantize(xt.cuda(), torch.from_numpy(gamma).cuda(), eps, ALL)
            torch.cuda.synchronize()
            assert_quant_equal(out, oracle_quant_fixed(y, ALL), f"adversarial eps={eps} {dtype}")


def test_rmsnorm_quantize_llm_shape_sampled_blocks():
    w = synth.workload("llm")
    pairs = synth.draw_sample_pairs(w.seed, w.B, w.H, 2)
    log(f"rmsnorm quantize llm {w.shape()} pairs {pairs}")
    x = synth.tensor_torch(w, "q", "cuda")
    gamma = _gamma(w.D, 7)
    out = mx.rmsnorm_quantize(x, gamma.cuda(), 1e-6, ALL)
    torch.cuda.synchronize()
    for b, h in pairs:
        xs = synth.head_slice_np(w, "q", b, h)
        for blk in (0, 101, w.S // 32 - 1):
            rows = slice(32 * blk, 32 * blk + 32)
            y = onorm.rmsnorm(xs[rows].double().numpy()[None, :, None, :], gamma.double().numpy(), 1e-6)
            sub = {}
            for lay, (d, s) in out.items():
                d = d[b:b + 1, rows, h:h + 1]
                s = s[b:b + 1, rows, h:h + 1] if lay == mx.ROW32 else s[b:b + 1, blk:blk + 1, h:h + 1]
                sub[lay] = (d.contiguous(), s.contiguous())
            assert_quant_equal(sub, oracle_quant_fixed(y, ALL), f"llm b{b} h{h} block {blk}")


def test_rmsnorm_quantize_varlen_exact():
    seqlens = [5, 128, 33, 200, 0, 64, 1]
    g = torch.Generator().manual_seed(4)
    x = (torch.randn(sum(seqlens), 3, 128, generator=g) * 4).to(torch.bfloat16).cuda()
    gamma = _gamma(128, 9)
    cu = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    log(f"rmsnorm quantize varlen T={cu[-1]}")
    out, csr = mx.rmsnorm_quantize_varlen(x, gamma.cuda(), torch.from_numpy(cu).cuda(), seqlens, 1e-6, ALL)
    torch.cuda.synchronize()
    assert np.array_equal(csr.cpu().numpy(), omx.padded_offsets(seqlens))
    y = onorm.rmsnorm(x.double().cpu().numpy(), gamma.double().numpy(), 1e-6)
    for h in range(3):
        ref = omx.quantize_varlen(y[:, h:h + 1], cu)
        for lay, key in ((mx.ROW32, "row32"), (mx.COL32, "col32"), (mx.SQ32, "sq32")):
            assert np.array_equal(to_np(out[lay][0])[:, h:h + 1], ref[key][0]), (key, h)
            assert np.array_equal(to_np(out[lay][1])[:, h:h + 1], ref[key][1]), (key, h)


def test_rmsnorm_quantize_rejects_bad_arguments():
    x = torch.randn(1, 32, 1, 64, device="cuda").to(torch.bfloat16)
    gamma = torch.ones(64, device="cuda")
    out = mx.alloc_quantized(x.shape, mx.ROW32, x.device)
    with pytest.raises(mx.MXError):
        mx.mx_rmsnorm_quantize(x, None, 1e-6, 1, 32, 1, 64, mx.ROW32, out[mx.ROW32][0], out[mx.ROW32][1],
                               None, None, None, None)
    with pytest.raises(mx.MXError):
        mx.mx_rmsnorm_quantize(x, gamma, -1.0, 1, 32, 1, 64, mx.ROW32, out[mx.ROW32][0], out[mx.ROW32][1],
                               None, None, None, None)
    with pytest.raises(mx.MXError):
        mx.mx_rmsnorm_quantize(x, gamma, float("nan"), 1, 32, 1, 64, mx.ROW32, out[mx.ROW32][0],
                               out[mx.ROW32][1], None, None, None, None)
