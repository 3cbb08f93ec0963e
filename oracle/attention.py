"""MXFP8 attention, forward and backward (CPU oracle, test infrastructure only).

Per (batch, head), as the pages describe it:
  * [Blog], "1. End-to-End Block-Scaled GEMM Fusion": both S = Q K^T and P V
    are products of MX-quantized operands.
  * [Blog], "2. Synchronized Online Softmax with Dynamic Scaling": the softmax
    runs in FP32 with the logits scaled by 1/sqrt(d_k) (the caller's
    softmax_scale, sigma).
  * [News], forward/backward paragraph: the FP32 softmax result P is converted
    to MXFP8 before P V, its block scales computed from the row maximum that
    the softmax already found; the backward quantizes Q, K and dO in square
    [32, 32] blocks, recomputes P, and re-quantizes the gradient dS online in
    transpose-invariant square blocks ([News], contributions paragraph);
    dQ is reduced in FP16 under a static power-of-two scale.

Readings taken where the pages are silent (each is listed in the design notes):
  * Log2-domain softmax with c = fl32(fl32(sigma) * fl32(log2 e)) and an
    integer row frame M = ceil(fl32(max_j S_ij * c)); p = fl32(exp2(fl32(S c - M))).
    A power-of-two frame leaves P's E4M3 codes independent of how a kernel
    tiles the key axis (MX quantization commutes with scaling by 2**k), so
    "reusing the max" gives a unique P-hat.
  * P-hat: blocks of 32 keys per query, aligned at key 0.  Normalizer l is the
    sum of the unquantized fp32 p.  O = (P-hat V-hat) / l.  LSE = ln2 (M + log2 l).
  * V enters P V with its blocks along the key axis (the contraction axis).
  * Backward: p = fl32(exp2(fl32(S' c - fl32(LSE * fl32(log2 e))))) from the
    forward's LSE; D_i = fl32(sum_d dO_id O_id) from the unquantized dO and O;
    dS = fl32(p * fl32(dP - D)); dS-hat in [32 queries x 32 keys] blocks;
    P-hat for dV = P^T dO in blocks of 32 queries per key; dK, dQ carry sigma.
  * Causal masking keeps keys j <= i (queries and keys have equal length).
  * The products whose values decide MX codes (S in the forward; S' and dP
    in the backward) accumulate as gfx950's block-scaled fp8 instruction
    does (``gemm="mfma"``, see oracle/gemm.py): the pages leave the MMA's
    internal precision open, and a code decided from S must be decided in
    the kernel's precision.  ``gemm="exact"`` gives the plain fl32(exact sum).
fl32 marks one rounding to float32; every other sum is float64.
"""
from __future__ import annotations

import math

import numpy as np

from . import gemm as gm
from . import mx
from . import mxsmall as ms

LOG2E32 = float(np.float32(math.log2(math.e)))


def fl32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16(x):
    """Round to bfloat16, nearest with ties to even, from the fp32 value (x is fp32-exact
    and finite): keep the top 16 bits of the fp32 pattern after adding 0x7FFF plus the
    lowest kept bit."""
    b = np.asarray(x, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def log2_scale(sigma: float) -> float:
    """c = fl32(fl32(sigma) * fl32(log2 e))."""
    return float(fl32(float(np.float32(sigma)) * LOG2E32))


def visible(Lq: int, Lk: int, causal: bool) -> np.ndarray:
    if not causal:
        return np.ones((Lq, Lk), dtype=bool)
    return np.arange(Lk)[None, :] <= np.arange(Lq)[:, None]


# ----------------------------------------------------------------- forward
def _quantize_qk(x, qk_fmt):
    """(dequantized values, element exponents) of a Q or K head [L, D] in ROW32 blocks: MXFP8
    E4M3, or MXFP6 / MXFP4 (qk_fmt "e2m3", "e3m2", "e2m1"; [News], paragraph on the block-scaled
    MMA's formats, read as the OCP MX v1.0 elements, see oracle/mxsmall.py)."""
    if qk_fmt == "e4m3":
        c, k = mx.quantize_row32(x)
        return mx.dequantize_row32(c, k), mx.element_exponent_row32(c, k)
    c, k = ms.quantize_rows(x, qk_fmt)
    return ms.dequantize_rows(c, k, qk_fmt), ms.element_exponent_rows(c, k, qk_fmt)


def forward_head(q, k, v, sigma, causal, quantize=True, exact=False, q_rows=None, gemm="mfma", p_round=None,
                 qk_fmt="e4m3"):
    """One (batch, head): q, k, v are [L, D] source values (fp32 or bf16 upcast).

    Returns a dict with O [L, D] (float64, before the output cast), LSE [L]
    (float64), the integer frame M, the normalizer l and the P-hat codes.
    ``quantize=False`` skips every MX step; ``exact=True`` skips every fp32
    rounding (used only to pin the oracle to textbook attention).
    ``q_rows`` (optional index array) computes only those query rows; every
    step is row-wise, so each returned row equals the full computation's.
    ``p_round="bf16"`` (with ``quantize=False``): the BF16 attention baseline, in
    which P enters P V rounded to bfloat16 and l still sums the fp32 p.
    ``qk_fmt``: element format of Q and K ("e4m3", or MXFP6 "e2m3" / "e3m2", MXFP4
    "e2m1"); P and V stay MXFP8 and every later step is unchanged.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    r = (lambda a: np.asarray(a, np.float64)) if exact else fl32
    if quantize:
        qh, qe = _quantize_qk(q, qk_fmt)
        kh, ke = _quantize_qk(k, qk_fmt)
        vh = mx.dequantize_col32(*mx.quantize_col32(v, axis=0), axis=0)
    else:
        qh, kh, vh = q, k, v
    c = sigma * math.log2(math.e) if exact else log2_scale(sigma)
    vis = visible(q.shape[0], k.shape[0], causal)
    if q_rows is not None:
        qh, vis = qh[q_rows], vis[q_rows]
        if quantize:
            qe = qe[q_rows]
    if quantize and not exact and gemm == "mfma":
        S = gm.matmul_mfma(qh, qe, kh, ke)
    else:
        S = r(qh @ kh.T)
    Smax = np.max(np.where(vis, S, -np.inf), axis=1)
    M = np.ceil(r(Smax * c))
    with np.errstate(over="ignore"):                  # masked entries may overflow; they are dropped
        p = r(np.exp2(r(S * c - M[:, None])))
    p = np.where(vis, p, 0.0)
    l = p.sum(axis=1)
    if quantize:
        pc, pk = mx.quantize_col32(p, axis=1)           # 32 keys per block, per query
        ph = mx.dequantize_col32(pc, pk, axis=1)
    else:
        pc, pk, ph = None, None, (bf16(p) if p_round == "bf16" else p)
    O = (ph @ vh) / l[:, None]
    LSE = math.log(2.0) * (M + np.log2(l))
    return {"O": O, "LSE": LSE, "M": M, "l": l, "P_codes": pc, "P_scales": pk, "S": S}


# ---------------------------------------------------------------- backward
def backward_head(q, k, v, o, do, lse, sigma, causal, quantize=True, exact=False, gemm="mfma", p_round=None):
    """One (batch, head) backward.  o, do: [L, D] (the forward output as the
    caller holds it, and the incoming gradient); lse: [L] (fp32 values).
    ``p_round="bf16"`` (with ``quantize=False``): the BF16 baseline, in which P
    (for dV) and dS (for dK and dQ) enter their products rounded to bfloat16.

    Returns float64 dQ, dK, dV [L, D] and the internals (p, dS, D).
    """
    q, k, v, o, do = (np.asarray(a, np.float64) for a in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    r = (lambda a: np.asarray(a, np.float64)) if exact else fl32
    if quantize:
        (qc, qk), (kc, kk), (dc, dk_) = mx.quantize_sq32(q, 0), mx.quantize_sq32(k, 0), mx.quantize_sq32(do, 0)
        vc, vk = mx.quantize_row32(v)
        qs, ks, dos = mx.dequantize_sq32(qc, qk, 0), mx.dequantize_sq32(kc, kk, 0), mx.dequantize_sq32(dc, dk_, 0)
        vr = mx.dequantize_row32(vc, vk)
        qe, ke, de = (mx.element_exponent_sq32(c_, k_, 0) for c_, k_ in ((qc, qk), (kc, kk), (dc, dk_)))
        ve = mx.element_exponent_row32(vc, vk)
    else:
        qs, ks, dos, vr = q, k, do, v
    use_mfma = quantize and not exact and gemm == "mfma"
    if exact:
        c, L2 = sigma * math.log2(math.e), lse * math.log2(math.e)
    else:
        c, L2 = log2_scale(sigma), fl32(lse * LOG2E32)
    vis = visible(q.shape[0], k.shape[0], causal)
    S = gm.matmul_mfma(qs, qe, ks, ke) if use_mfma else r(qs @ ks.T)
    with np.errstate(over="ignore"):                  # masked entries may overflow; they are dropped
        p = np.where(vis, r(np.exp2(r(S * c - L2[:, None]))), 0.0)
    dP = gm.matmul_mfma(dos, de, vr, ve) if use_mfma else r(dos @ vr.T)
    Dv = r(np.sum(do * o, axis=1))
    dS = np.where(vis, r(p * r(dP - Dv[:, None])), 0.0)
    if quantize:
        dSh = mx.dequantize_sq32(*mx.quantize_sq32(dS, 0), 0)   # [32 q x 32 k] blocks
        pb = mx.dequantize_col32(*mx.quantize_col32(p, axis=0), axis=0)  # 32 queries per key
    elif p_round == "bf16":
        dSh, pb = bf16(dS), bf16(p)
    else:
        dSh, pb = dS, p
    dV = pb.T @ dos
    dK = sigma * (dSh.T @ qs)
    dQ = sigma * (dSh @ ks)
    return {"dQ": dQ, "dK": dK, "dV": dV, "p": p, "dS": dS, "D": Dv, "S": S, "dP": dP}


def backward_head_blocks(q, k, v, o, do, lse, sigma, causal, q_blocks=(), k_blocks=()):
    """backward_head (MX quantization, the instruction's accumulation for S and dP) for selected
    32-row blocks only: dQ of the query blocks in q_blocks and dK, dV of the key blocks in
    k_blocks.  Every step is local to such a block: the square [32 x 32] dS blocks of one query
    block need only that block's rows against all keys, and P's 32-query blocks and dS's blocks of
    one key block need all queries against only that block's keys.  The MX operands, D and the
    frame are formed exactly as in backward_head, so each returned block equals the corresponding
    rows of its full result.  Returns {"dQ": {qb: [rows, D]}, "dK": {kb: ...}, "dV": {kb: ...}}."""
    q, k, v, o, do = (np.asarray(a, np.float64) for a in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    L = q.shape[0]
    (qc, qk), (kc, kk), (dc, dk_) = mx.quantize_sq32(q, 0), mx.quantize_sq32(k, 0), mx.quantize_sq32(do, 0)
    vc, vk = mx.quantize_row32(v)
    qs, ks, dos = mx.dequantize_sq32(qc, qk, 0), mx.dequantize_sq32(kc, kk, 0), mx.dequantize_sq32(dc, dk_, 0)
    vr = mx.dequantize_row32(vc, vk)
    qe, ke, de = (mx.element_exponent_sq32(c_, k_, 0) for c_, k_ in ((qc, qk), (kc, kk), (dc, dk_)))
    ve = mx.element_exponent_row32(vc, vk)
    c, L2 = log2_scale(sigma), fl32(lse * LOG2E32)
    Dv = fl32(np.sum(do * o, axis=1))

    def p_ds(ri, cj):
        vis = visible(L, L, causal)[np.ix_(ri, cj)] if causal else np.ones((len(ri), len(cj)), bool)
        S = gm.matmul_mfma(qs[ri], qe[ri], ks[cj], ke[cj])
        with np.errstate(over="ignore"):
            p = np.where(vis, fl32(np.exp2(fl32(S * c - L2[ri, None]))), 0.0)
        dP = gm.matmul_mfma(dos[ri], de[ri], vr[cj], ve[cj])
        return p, np.where(vis, fl32(p * fl32(dP - Dv[ri, None])), 0.0)

    everything = np.arange(L)
    out = {"dQ": {}, "dK": {}, "dV": {}}
    for qb in q_blocks:
        ri = np.arange(32 * qb, min(L, 32 * qb + 32))
        _, dS = p_ds(ri, everything)
        dSh = mx.dequantize_sq32(*mx.quantize_sq32(dS, 0), 0)          # one query block, all key blocks
        out["dQ"][qb] = sigma * (dSh @ ks)
    for kb in k_blocks:
        cj = np.arange(32 * kb, min(L, 32 * kb + 32))
        p, dS = p_ds(everything, cj)
        dSh = mx.dequantize_sq32(*mx.quantize_sq32(dS, 0), 0)          # all query blocks, one key block
        pb = mx.dequantize_col32(*mx.quantize_col32(p, axis=0), axis=0)  # 32 queries per key
        out["dV"][kb] = pb.T @ dos
        out["dK"][kb] = sigma * (dSh.T @ qs)
    return out


# -------------------------------------------------------- textbook, float64
def attention_fp64(q, k, v, sigma, causal):
    """softmax(sigma q k^T) v in float64, no quantization; returns (O, LSE)."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    S = sigma * (q @ k.T)
    S = np.where(visible(q.shape[0], k.shape[0], causal), S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    e = np.exp(S - m)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ v, (m + np.log(l))[:, 0]


def attention_fp64_backward(q, k, v, do, sigma, causal):
    """Analytic gradients of attention_fp64 with respect to q, k, v."""
    q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
    S = sigma * (q @ k.T)
    S = np.where(visible(q.shape[0], k.shape[0], causal), S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P = P / P.sum(axis=1, keepdims=True)
    dV = P.T @ do
    dP = do @ v.T
    dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
    return sigma * (dS @ k), sigma * (dS.T @ q), dV


# ------------------------------------------------------- whole-tensor views
def _heads(x, cu_seqlens):
    """Yield (key, [L, D] view) per (batch, head) or (sequence, head)."""
    if cu_seqlens is None:
        B, S, H, D = x.shape
        for b in range(B):
            for h in range(H):
                yield (b, h), x[b, :, h, :]
    else:
        T, H, D = x.shape
        for s in range(len(cu_seqlens) - 1):
            for h in range(H):
                yield (s, h), x[cu_seqlens[s]:cu_seqlens[s + 1], h, :]


def mx_attention_forward(q, k, v, sigma, causal, cu_seqlens=None, bf16_baseline=False, qk_fmt="e4m3"):
    """Forward over [B, S, H, D] (or packed [T, H, D] with cu_seqlens).

    Returns O (float64, q's shape) and LSE ([B, H, S] or [H, T], float64).
    ``bf16_baseline``: no MX step, P rounded to bfloat16 before P V (the BF16
    attention the pages compare against, [News] headline figures).
    ``qk_fmt``: element format of Q and K (see forward_head).
    """
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    O = np.zeros_like(q)
    if cu_seqlens is None:
        LSE = np.zeros((q.shape[0], q.shape[2], q.shape[1]))
    else:
        LSE = np.zeros((q.shape[1], q.shape[0]))
    ks, vs = dict(_heads(k, cu_seqlens)), dict(_heads(v, cu_seqlens))
    for key, qh in _heads(q, cu_seqlens):
        if qh.shape[0] == 0:
            continue
        res = (forward_head(qh, ks[key], vs[key], sigma, causal, quantize=False, p_round="bf16")
               if bf16_baseline else forward_head(qh, ks[key], vs[key], sigma, causal, qk_fmt=qk_fmt))
        a, h = key
        if cu_seqlens is None:
            O[a, :, h, :] = res["O"]
            LSE[a, h, :] = res["LSE"]
        else:
            O[cu_seqlens[a]:cu_seqlens[a + 1], h, :] = res["O"]
            LSE[h, cu_seqlens[a]:cu_seqlens[a + 1]] = res["LSE"]
    return O, LSE


def mx_attention_backward(q, k, v, o, do, lse, sigma, causal, cu_seqlens=None, bf16_baseline=False):
    """Backward over whole tensors; lse is [B, H, S] (or [H, T]).  Returns float64 dQ, dK, dV.
    ``bf16_baseline``: no MX step, P and dS rounded to bfloat16 before their products."""
    q, k, v, o, do = (np.asarray(a, np.float64) for a in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    K, V, Oh, DOh = (dict(_heads(t, cu_seqlens)) for t in (k, v, o, do))
    for key, qh in _heads(q, cu_seqlens):
        if qh.shape[0] == 0:
            continue
        a, h = key
        if cu_seqlens is None:
            lh = lse[a, h, :]
            sl = (a, slice(None), h, slice(None))
        else:
            lh = lse[h, cu_seqlens[a]:cu_seqlens[a + 1]]
            sl = (slice(cu_seqlens[a], cu_seqlens[a + 1]), h, slice(None))
        res = (backward_head(qh, K[key], V[key], Oh[key], DOh[key], lh, sigma, causal, quantize=False,
                             p_round="bf16") if bf16_baseline
               else backward_head(qh, K[key], V[key], Oh[key], DOh[key], lh, sigma, causal))
        dQ[sl], dK[sl], dV[sl] = res["dQ"], res["dK"], res["dV"]
    return dQ, dK, dV
