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


def check_out_bounds(o_gpu, lo, hi, o_exact, what, bf16=False, rel=1e-3, max_ref=None):
    """The parity check of a several-valued O: every element inside the oracle's admissible
    interval [lo, hi] (oracle/attention.py forward_head_bounds) within rel * max|O| (+ half a bf16
    ulp for bf16 outputs).  Where the interval is a single value this is the plain check against
    the exact oracle.  Logs how many rows differ from the exact oracle by more than the plain
    tolerance, i.e. needed the widening (a row whose P codes moved with the product's rounding)."""
    o_gpu = np.asarray(o_gpu, np.float64)
    tol = rel * (np.max(np.abs(o_exact)) if max_ref is None else max_ref)
    slack = tol + (bf16_half_ulp(np.maximum(np.abs(lo), np.abs(hi))) * (1 + 2.0 ** -7) if bf16 else 0.0)
    excess = np.maximum(np.maximum(lo - o_gpu, o_gpu - hi), 0.0)
    worst = float(np.max(excess - slack)) if excess.size else 0.0
    err = np.abs(o_gpu - o_exact)
    plain = err > tol + (bf16_half_ulp(o_exact) * (1 + 2.0 ** -7) if bf16 else 0.0)
    rows = int(np.sum(np.any(plain.reshape(-1, o_gpu.shape[-1]), axis=1)))
    wide = float(np.mean((hi - lo) > tol)) if lo.size else 0.0
    log(f"  {what}: max|O - O_exact| {np.max(err):.3e} tol {tol:.3e}; rows beyond the plain bound {rows} of "
        f"{err.size // err.shape[-1]}; max excess over the admissible interval {np.max(excess):.3e}; "
        f"{100 * wide:.2f}% of elements with an interval wider than the tolerance")
    assert worst <= 0, f"{what}: O leaves the admissible interval by {worst:.3e} beyond the tolerance {tol:.3e}"
    return rows


def check_lse_bounds(l_gpu, lo, hi, what):
    l_gpu = np.asarray(l_gpu, np.float64)
    bound = 1e-4 + 1e-6 * np.maximum(np.abs(lo), np.abs(hi))
    excess = np.maximum(np.maximum(lo - l_gpu, l_gpu - hi), 0.0)
    log(f"  {what}: max LSE excess over the admissible interval {np.max(excess):.3e}")
    assert np.all(excess <= bound), f"{what}: LSE leaves the admissible interval by {np.max(excess - bound):.3e}"


def check_grad_bounds(g, lo, hi, exact, what, tol=5e-3):
    """The parity check of a several-valued gradient: the part of the GPU result outside the
    oracle's admissible interval (oracle/attention.py backward_bounds) must stay within tol relative
    Frobenius error of the exact oracle's gradient.  Logs the plain relative error too."""
    g = np.asarray(g, np.float64)
    excess = np.maximum(np.maximum(lo - g, g - hi), 0.0)
    nrm = np.linalg.norm(exact)
    e = float(np.linalg.norm(excess) / nrm) if nrm > 0 else float(np.linalg.norm(excess))
    plain = float(np.linalg.norm(g - exact) / nrm) if nrm > 0 else float(np.linalg.norm(g - exact))
    width = float(np.linalg.norm(hi - lo) / nrm) if nrm > 0 else 0.0
    log(f"  {what}: rel Frobenius vs exact {plain:.2e}; excess over the admissible interval {e:.2e}; "
        f"interval width (rel Frobenius) {width:.2e}")
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    assert e <= tol, f"{what}: rel Frobenius excess {e:.3e} > {tol}"
    return plain


def check_lse(l_gpu, l_ref, what):
    err = np.abs(np.asarray(l_gpu, np.float64) - l_ref)
    bound = 1e-4 + 1e-6 * np.abs(l_ref)
    log(f"  {what}: max|dLSE| {np.max(err):.3e}")
    assert np.all(err <= bound), f"{what}: LSE error {np.max(err - bound):.3e} over bound"


def rel_fro(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


def oracle_forward_head(q, k, v, sigma, causal, chunk=1024):
    """The oracle forward of one head in row chunks (each chunk's causal key range only: the
    quantization of K and V is local to rows and to 32-key blocks, so every row equals
    forward_head's).  Returns (O as bf16-rounded float64, LSE as fp32-rounded float64): the bytes
    a caller would hold and pass to the backward."""
    L = q.shape[0]
    O = np.zeros(q.shape)
    LSE = np.zeros(L)
    for r0 in range(0, L, chunk):
        r1 = min(L, r0 + chunk)
        n = r1 if causal else L
        r = at.forward_head(q[:n], k[:n], v[:n], sigma, causal, q_rows=np.arange(r0, r1))
        O[r0:r1], LSE[r0:r1] = r["O"], r["LSE"]
    return at.bf16(O), at.fl32(LSE)
