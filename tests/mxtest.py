"""Shared helpers for the GPU parity tests (inputs, oracle calls, checks)."""
import math

import numpy as np
import torch

import mxfp8_block_scaled_flash_amd as mx
import synth
from oracle import attention as at
from oracle import mx as omx


def log(*a):
    print(*a, flush=True)


def to_np(t):
    return t.detach().cpu().double().numpy() if t.dtype != torch.uint8 else t.detach().cpu().numpy()


def oracle_quant_fixed(x_np, layouts):
    """Oracle codes/scales for a [B, S, H, D] array, in the ABI's layouts."""
    out = {}
    if layouts & mx.ROW32:
        out[mx.ROW32] = omx.quantize_row32(x_np)
    if layouts & mx.COL32:
        out[mx.COL32] = omx.quantize_col32(x_np, axis=1)
    if layouts & mx.SQ32:
        out[mx.SQ32] = omx.quantize_sq32(x_np, 1)
    return out


def assert_quant_equal(gpu, ref, what=""):
    for lay, (codes, scales) in ref.items():
        gd, gs = to_np(gpu[lay][0]), to_np(gpu[lay][1])
        name = mx.LAYOUT_NAMES[lay]
        assert gd.shape == codes.shape and gs.shape == scales.shape, (what, name, gd.shape, codes.shape)
        nd = int(np.sum(gd != codes))
        ns = int(np.sum(gs != scales))
        if nd or ns:
            idx = np.argwhere(gd != codes)[:5]
            raise AssertionError(f"{what} {name}: {nd} payload and {ns} scale mismatches; first payload "
                                 f"mismatches at {idx.tolist()}: gpu {[int(gd[tuple(i)]) for i in idx]} "
                                 f"oracle {[int(codes[tuple(i)]) for i in idx]}")


def bf16_half_ulp(x):
    """Half a bf16 ulp of |x| (elementwise)."""
    a = np.abs(x)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 8)


def check_out(o_gpu, o_ref, what, bf16=False, rel=1e-3):
    """max|dO| <= rel * max|O_ref|  (+ half a bf16 ulp of O_ref for bf16 outputs)."""
    o_gpu = np.asarray(o_gpu, np.float64)
    tol = rel * np.max(np.abs(o_ref))
    err = np.abs(o_gpu - o_ref)
    bound = tol + (bf16_half_ulp(o_ref) * (1 + 2.0 ** -7) if bf16 else 0.0)
    worst = float(np.max(err - bound))
    log(f"  {what}: max|dO| {np.max(err):.3e}  tol {tol:.3e}  max|O| {np.max(np.abs(o_ref)):.3e}")
    assert worst <= 0, f"{what}: |dO| exceeds bound by {worst:.3e} (max err {np.max(err):.3e}, tol {tol:.3e})"


def check_lse(l_gpu, l_ref, what):
    err = np.abs(np.asarray(l_gpu, np.float64) - l_ref)
    bound = 1e-4 + 1e-6 * np.abs(l_ref)
    log(f"  {what}: max|dLSE| {np.max(err):.3e}")
    assert np.all(err <= bound), f"{what}: LSE error {np.max(err - bound):.3e} over bound"


def rel_fro(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))
