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
  * Every product of MX operands is the exact sum rounded once to fp32
    (oracle/gemm.py).  The pages leave the matrix unit's internal precision
    open, so a kernel's product may differ from that value by up to the
    stated bound eps; codes decided from such a product (P, dS) are then
    several-valued.  ``forward_head_bounds`` and ``backward_bounds`` give the
    set of admissible results: the same steps, in the same order, on
    intervals that hold every value an eps-close product can lead to.
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


# ------------------------------------------------------------- MX operands
def _quantize_qk(x, qk_fmt):
    """(dequantized values, element magnitudes) of a Q or K head [L, D] in ROW32 blocks: MXFP8
    E4M3, or MXFP6 / MXFP4 (qk_fmt "e2m3", "e3m2", "e2m1"; [News], paragraph on the block-scaled
    MMA's formats, read as the OCP MX v1.0 elements, see oracle/mxsmall.py)."""
    if qk_fmt == "e4m3":
        c, k = mx.quantize_row32(x)
        vals = mx.dequantize_row32(c, k)
        return vals, gm.magnitudes(vals, mx.element_exponent_row32(c, k))
    c, k = ms.quantize_rows(x, qk_fmt)
    vals = ms.dequantize_rows(c, k, qk_fmt)
    return vals, gm.magnitudes(vals, ms.element_exponent_rows(c, k, qk_fmt))


def _quantize_keys(x):
    """V for P V: blocks of 32 keys per feature (COL32 along the key axis); (values, magnitudes)."""
    c, k = mx.quantize_col32(x, axis=0)
    vals = mx.dequantize_col32(c, k, axis=0)
    return vals, gm.magnitudes(vals, mx.element_exponent_col32(c, k, axis=0))


def _quantize_sq(x, fmt="e4m3"):
    """Square [32 tokens x 32 features] blocks (Q, K, dO in the backward); (values, magnitudes).
    fmt: MXFP8 E4M3, or for Q and K the MXFP6 / MXFP4 elements (oracle/mxsmall.py)."""
    if fmt == "e4m3":
        c, k = mx.quantize_sq32(x, 0)
        vals = mx.dequantize_sq32(c, k, 0)
        return vals, gm.magnitudes(vals, mx.element_exponent_sq32(c, k, 0))
    c, k = ms.quantize_sq32(x, fmt)
    vals = ms.dequantize_sq32(c, k, fmt)
    return vals, gm.magnitudes(vals, ms.element_exponent_sq32(c, k, fmt))


def _quantize_row(x):
    """V for dP = dO V^T: blocks of 32 features (ROW32); (values, magnitudes)."""
    c, k = mx.quantize_row32(x)
    vals = mx.dequantize_row32(c, k)
    return vals, gm.magnitudes(vals, mx.element_exponent_row32(c, k))


# ----------------------------------------------------------------- forward
def forward_head(q, k, v, sigma, causal, quantize=True, exact=False, q_rows=None, p_round=None,
                 qk_fmt="e4m3", s_delta=None):
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
    ``s_delta`` (tests only): added to the exact sum before its fp32 rounding, standing for a
    matrix unit whose product differs from the exact one (rows as selected by q_rows).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    r = (lambda a: np.asarray(a, np.float64)) if exact else fl32
    if quantize:
        qh, _ = _quantize_qk(q, qk_fmt)
        kh, _ = _quantize_qk(k, qk_fmt)
        vh, _ = _quantize_keys(v)
    else:
        qh, kh, vh = q, k, v
    c = sigma * math.log2(math.e) if exact else log2_scale(sigma)
    vis = visible(q.shape[0], k.shape[0], causal)
    if q_rows is not None:
        qh, vis = qh[q_rows], vis[q_rows]
    prod = qh @ kh.T
    if s_delta is not None:
        prod = prod + s_delta
    S = r(prod)
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


# fp32 slack of an implementation's own roundings, used only by the *_bounds functions: the exp2
# argument is rounded once at a magnitude below |S c| + |frame| + 10 (a lazily moved integer frame
# stays within 10 of the final one), exp2 is good to 2 ulps, and an fp32 sum of n terms is within
# n 2^-24 of its exact value.
def _exp2_rel(Sc, frame):
    return math.log(2.0) * 2.0 ** -23 * (np.abs(Sc) + np.abs(frame) + 10.0) + 2.0 ** -21


def forward_head_bounds(q, k, v, sigma, causal, q_rows=None, qk_fmt="e4m3", mma=True, fp32=True):
    """The admissible O and LSE of one (batch, head): forward_head's steps on intervals.

    A kernel whose products lie within oracle/gemm.py's bound eps of the exact sums
    (``mma=True``) and whose own fp32 roundings are ordinary (``fp32=True``) returns an O inside
    [O_lo, O_hi] up to the accumulation order of its P V sums, and an LSE inside [LSE_lo, LSE_hi]:
      * S within eps (+ half an fp32 ulp) -> p = 2^(S c - M) within [p_lo, p_hi] in the frame M of
        the exact S (any other integer frame scales p, l and P^'s scales by the same power of two);
      * P^ = MX rounding of p in blocks of 32 keys: oracle/mx.py round_interval;
      * O = (P^ V^) / l with P^ >= 0 and l = sum p > 0, plus eps of the P V product.
    With mma=False and fp32=False the bounds collapse onto forward_head's O and LSE.
    Returns dict O_lo, O_hi, LSE_lo, LSE_hi (rows as selected by q_rows)."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    qh, qm = _quantize_qk(q, qk_fmt)
    kh, km = _quantize_qk(k, qk_fmt)
    vh, vm = _quantize_keys(v)
    c = log2_scale(sigma)
    vis = visible(q.shape[0], k.shape[0], causal)
    if q_rows is not None:
        qh, qm, vis = qh[q_rows], qm[q_rows], vis[q_rows]
    S = fl32(qh @ kh.T)
    eps = gm.product_error_bound(qm, km) + 2.0 ** -24 * np.abs(S) if mma else 0.0
    M = np.ceil(fl32(np.max(np.where(vis, S, -np.inf), axis=1) * c))[:, None]
    with np.errstate(over="ignore"):
        if fp32:
            rel = _exp2_rel(S * c, M)
            p_lo = np.where(vis, np.exp2((S - eps) * c - M) * (1 - rel), 0.0)
            p_hi = np.where(vis, np.exp2((S + eps) * c - M) * (1 + rel), 0.0)
        else:                                           # forward_head's own roundings
            p_lo = np.where(vis, fl32(np.exp2(fl32((S - eps) * c - M))), 0.0)
            p_hi = np.where(vis, fl32(np.exp2(fl32((S + eps) * c - M))), 0.0)
    P_lo, P_hi, P_k = mx.round_interval(p_lo, p_hi, 1, mx.BLOCK)
    vp, vn = np.maximum(vh, 0.0), np.minimum(vh, 0.0)
    N_lo = P_lo @ vp + P_hi @ vn
    N_hi = P_hi @ vp + P_lo @ vn
    if mma:
        P_mag = np.where(P_hi > 0, np.maximum(P_hi, np.exp2(P_k - 133.0)), 0.0)
        e_o = gm.product_error_bound(P_mag, vm.T)
        N_lo, N_hi = N_lo - e_o, N_hi + e_o
    n = vis.sum(axis=1)
    l_lo = p_lo.sum(axis=1) * ((1 - n * 2.0 ** -24) if fp32 else 1.0)
    l_hi = p_hi.sum(axis=1) * ((1 + n * 2.0 ** -24) if fp32 else 1.0)
    O_lo = np.minimum(N_lo / l_lo[:, None], N_lo / l_hi[:, None])
    O_hi = np.maximum(N_hi / l_lo[:, None], N_hi / l_hi[:, None])
    return {"O_lo": O_lo, "O_hi": O_hi, "LSE_lo": math.log(2.0) * (M[:, 0] + np.log2(l_lo)),
            "LSE_hi": math.log(2.0) * (M[:, 0] + np.log2(l_hi))}


# ---------------------------------------------------------------- backward
def backward_head(q, k, v, o, do, lse, sigma, causal, quantize=True, exact=False, p_round=None,
                  s_delta=None, dp_delta=None, qk_fmt="e4m3"):
    """One (batch, head) backward.  o, do: [L, D] (the forward output as the
    caller holds it, and the incoming gradient); lse: [L] (fp32 values).
    ``p_round="bf16"`` (with ``quantize=False``): the BF16 baseline, in which P
    (for dV) and dS (for dK and dQ) enter their products rounded to bfloat16.
    ``s_delta``, ``dp_delta`` (tests only): added to the exact sums of S' and dP before their
    fp32 rounding (see forward_head).
    ``qk_fmt``: element format of Q and K in their square blocks ("e4m3", or MXFP6 "e2m3" /
    "e3m2", MXFP4 "e2m1"); dO, V, P and dS stay MXFP8.

    Returns float64 dQ, dK, dV [L, D] and the internals (p, dS, D).
    """
    q, k, v, o, do = (np.asarray(a, np.float64) for a in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    r = (lambda a: np.asarray(a, np.float64)) if exact else fl32
    if quantize:
        (qs, _), (ks, _), (dos, _) = _quantize_sq(q, qk_fmt), _quantize_sq(k, qk_fmt), _quantize_sq(do)
        vr, _ = _quantize_row(v)
    else:
        qs, ks, dos, vr = q, k, do, v
    if exact:
        c, L2 = sigma * math.log2(math.e), lse * math.log2(math.e)
    else:
        c, L2 = log2_scale(sigma), fl32(lse * LOG2E32)
    vis = visible(q.shape[0], k.shape[0], causal)
    S = r(qs @ ks.T + (0.0 if s_delta is None else s_delta))
    with np.errstate(over="ignore"):                  # masked entries may overflow; they are dropped
        p = np.where(vis, r(np.exp2(r(S * c - L2[:, None]))), 0.0)
    dP = r(dos @ vr.T + (0.0 if dp_delta is None else dp_delta))
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


def _rows_of(blocks, L):
    return np.concatenate([np.arange(32 * b, min(L, 32 * b + 32)) for b in blocks]) if len(blocks) else \
        np.zeros(0, np.int64)


def backward_head_blocks(q, k, v, o, do, lse, sigma, causal, q_blocks=(), k_blocks=(), qk_fmt="e4m3"):
    """backward_head for selected 32-row blocks only: dQ of the query blocks in q_blocks and dK, dV
    of the key blocks in k_blocks.  Every step is local to such a block: the square [32 x 32] dS
    blocks of one query block need only that block's rows against all keys, and P's 32-query blocks
    and dS's blocks of one key block need all queries against only that block's keys.  The MX
    operands, D and the products are formed exactly as in backward_head, so each returned block
    equals the corresponding rows of its full result.
    Returns {"dQ": {qb: [rows, D]}, "dK": {kb: ...}, "dV": {kb: ...}}."""
    q, k, v, o, do = (np.asarray(a, np.float64) for a in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    L = q.shape[0]
    (qs, _), (ks, _), (dos, _) = _quantize_sq(q, qk_fmt), _quantize_sq(k, qk_fmt), _quantize_sq(do)
    vr, _ = _quantize_row(v)
    c, L2 = log2_scale(sigma), fl32(lse * LOG2E32)
    Dv = fl32(np.sum(do * o, axis=1))

    def p_ds(ri, cj):
        vis = visible(L, L, causal)[np.ix_(ri, cj)]
        S = fl32(qs[ri] @ ks[cj].T)
        with np.errstate(over="ignore"):
            p = np.where(vis, fl32(np.exp2(fl32(S * c - L2[ri, None]))), 0.0)
        dP = fl32(dos[ri] @ vr[cj].T)
        return p, np.where(vis, fl32(p * fl32(dP - Dv[ri, None])), 0.0)

    everything = np.arange(L)
    out = {"dQ": {}, "dK": {}, "dV": {}}
    for qb in q_blocks:
        ri = _rows_of([qb], L)
        _, dS = p_ds(ri, everything)
        dSh = mx.dequantize_sq32(*mx.quantize_sq32(dS, 0), 0)          # one query block, all key blocks
        out["dQ"][qb] = sigma * (dSh @ ks)
    for kb in k_blocks:
        cj = _rows_of([kb], L)
        p, dS = p_ds(everything, cj)
        dSh = mx.dequantize_sq32(*mx.quantize_sq32(dS, 0), 0)          # all query blocks, one key block
        pb = mx.dequantize_col32(*mx.quantize_col32(p, axis=0), axis=0)  # 32 queries per key
        out["dV"][kb] = pb.T @ dos
        out["dK"][kb] = sigma * (dSh.T @ qs)
    return out


def _runs(blocks, chunk):
    """Split a list of block indices into runs of at most ``chunk`` consecutive blocks."""
    runs, cur = [], []
    for b in blocks:
        if cur and (b != cur[-1] + 1 or len(cur) == chunk):
            runs.append(cur)
            cur = []
        cur.append(b)
    if cur:
        runs.append(cur)
    return runs


def _interval_matmul(a_lo, a_hi, b):
    """[lo, hi] of A @ b for A anywhere in [a_lo, a_hi] elementwise and b fixed."""
    bp, bn = np.maximum(b, 0.0), np.minimum(b, 0.0)
    return a_lo @ bp + a_hi @ bn, a_hi @ bp + a_lo @ bn


def backward_bounds(q, k, v, o, do, lse, sigma, causal, q_blocks=None, k_blocks=None, mma=True, fp32=True,
                    chunk=8, qk_fmt="e4m3"):
    """The admissible dQ (rows of q_blocks), dK and dV (rows of k_blocks) of one (batch, head):
    backward_head's steps on intervals, as forward_head_bounds does for the forward.
      * S' and dP within eps of their exact sums -> p = 2^(S' c - LSE log2 e) in [p_lo, p_hi];
        D = sum dO O within its fp32 summation slack; dS = p (dP - D) by interval products;
      * dS^ (square 32 x 32 blocks) and P^ for dV (32 queries per key): round_interval;
      * dV = P^T dO^, dK = sigma dS^T Q^, dQ = sigma dS^ K^ by interval sums, plus eps of each
        product.
    The fp16 reduction of dQ under its static scale is an approximation the comparison tolerance
    covers, not part of the bounds.  With mma=False and fp32=False the bounds collapse onto
    backward_head_blocks.  q_blocks / k_blocks: 32-row block indices (None: all).
    Returns {"dQ": (lo, hi), "dK": (lo, hi), "dV": (lo, hi), "q_rows": rows, "k_rows": rows}."""
    q, k, v, o, do = (np.asarray(a, np.float64) for a in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    L, D = q.shape
    nb = (L + 31) // 32
    q_blocks = list(range(nb)) if q_blocks is None else list(q_blocks)
    k_blocks = list(range(nb)) if k_blocks is None else list(k_blocks)
    (qs, qm), (ks, km), (dos, dm) = _quantize_sq(q, qk_fmt), _quantize_sq(k, qk_fmt), _quantize_sq(do)
    vr, vm = _quantize_row(v)
    c, L2 = log2_scale(sigma), fl32(lse * LOG2E32)
    Dv = fl32(np.sum(do * o, axis=1))
    eD = 2.0 ** -17 * np.sum(np.abs(do * o), axis=1) if fp32 else 0.0
    def intervals(ri, cj):
        vis = visible(L, L, causal)[np.ix_(ri, cj)]
        S = fl32(qs[ri] @ ks[cj].T)
        dP = fl32(dos[ri] @ vr[cj].T)
        eS = gm.product_error_bound(qm[ri], km[cj]) + 2.0 ** -24 * np.abs(S) if mma else 0.0
        eP = gm.product_error_bound(dm[ri], vm[cj]) + 2.0 ** -24 * np.abs(dP) if mma else 0.0
        a = S * c - L2[ri, None]
        Di = Dv[ri, None]
        with np.errstate(over="ignore"):
            if fp32:
                rel = _exp2_rel(S * c, L2[ri, None])
                p_lo = np.where(vis, np.exp2(a - eS * c) * (1 - rel), 0.0)
                p_hi = np.where(vis, np.exp2(a + eS * c) * (1 + rel), 0.0)
                x_lo = (dP - eP) - (Di + eD[ri, None])
                x_hi = (dP + eP) - (Di - eD[ri, None])
                x_lo, x_hi = x_lo - 2.0 ** -24 * np.abs(x_lo), x_hi + 2.0 ** -24 * np.abs(x_hi)
            else:                                       # backward_head's own roundings
                p_lo = np.where(vis, fl32(np.exp2(fl32(S * c - eS * c - L2[ri, None]))), 0.0)
                p_hi = np.where(vis, fl32(np.exp2(fl32(S * c + eS * c - L2[ri, None]))), 0.0)
                x_lo, x_hi = fl32(dP - eP - Di), fl32(dP + eP - Di)
        s_lo = np.where(vis, np.minimum(p_lo * x_lo, p_hi * x_lo), 0.0)
        s_hi = np.where(vis, np.maximum(p_lo * x_hi, p_hi * x_hi), 0.0)
        if fp32:
            s_lo, s_hi = s_lo - 2.0 ** -24 * np.abs(s_lo), s_hi + 2.0 ** -24 * np.abs(s_hi)
        else:
            s_lo, s_hi = fl32(s_lo), fl32(s_hi)
        return p_lo, p_hi, s_lo, s_hi

    def mag(lo, hi, kcode):
        a = np.maximum(np.abs(lo), np.abs(hi))
        return np.where(a > 0, np.maximum(a, np.exp2(kcode - 133.0)), 0.0)

    everything = np.arange(L)
    out = {"q_rows": _rows_of(q_blocks, L), "k_rows": _rows_of(k_blocks, L)}
    parts = []
    for run in _runs(q_blocks, chunk):               # consecutive query blocks: whole square blocks
        ri = _rows_of(run, L)
        _, _, s_lo, s_hi = intervals(ri, everything)
        qlo, qhi, kk = mx.round_interval(s_lo, s_hi, mx.BLOCK, mx.BLOCK)
        lo, hi = _interval_matmul(qlo, qhi, ks)
        if mma:
            e = gm.product_error_bound(mag(qlo, qhi, kk), km.T)
            lo, hi = lo - e, hi + e
        parts.append((sigma * lo, sigma * hi))
    out["dQ"] = (np.concatenate([a for a, _ in parts]) if parts else np.zeros((0, D)),
                 np.concatenate([b for _, b in parts]) if parts else np.zeros((0, D)))
    dk, dv = [], []
    for run in _runs(k_blocks, chunk):               # consecutive key blocks: whole square blocks
        cj = _rows_of(run, L)
        p_lo, p_hi, s_lo, s_hi = intervals(everything, cj)
        slo, shi, sk = mx.round_interval(s_lo, s_hi, mx.BLOCK, mx.BLOCK)
        plo, phi, pk = mx.round_interval(p_lo, p_hi, mx.BLOCK, 1)
        klo, khi = _interval_matmul(slo.T, shi.T, qs)
        vlo, vhi = _interval_matmul(plo.T, phi.T, dos)
        if mma:
            ek = gm.product_error_bound(mag(slo, shi, sk).T, qm.T)
            ev = gm.product_error_bound(mag(plo, phi, pk).T, dm.T)
            klo, khi, vlo, vhi = klo - ek, khi + ek, vlo - ev, vhi + ev
        dk.append((sigma * klo, sigma * khi))
        dv.append((vlo, vhi))
    out["dK"] = (np.concatenate([a for a, _ in dk]) if dk else np.zeros((0, D)),
                 np.concatenate([b for _, b in dk]) if dk else np.zeros((0, D)))
    out["dV"] = (np.concatenate([a for a, _ in dv]) if dv else np.zeros((0, D)),
                 np.concatenate([b for _, b in dv]) if dv else np.zeros((0, D)))
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


def mx_attention_backward(q, k, v, o, do, lse, sigma, causal, cu_seqlens=None, bf16_baseline=False, qk_fmt="e4m3"):
    """Backward over whole tensors; lse is [B, H, S] (or [H, T]).  Returns float64 dQ, dK, dV.
    ``bf16_baseline``: no MX step, P and dS rounded to bfloat16 before their products.
    ``qk_fmt``: element format of Q and K (backward_head)."""
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
               else backward_head(qh, K[key], V[key], Oh[key], DOh[key], lh, sigma, causal, qk_fmt=qk_fmt))
        dQ[sl], dK[sl], dV[sl] = res["dQ"], res["dK"], res["dV"]
    return dQ, dK, dV


def mx_attention_forward_bounds(q, k, v, sigma, causal, cu_seqlens=None, qk_fmt="e4m3"):
    """forward_head_bounds over whole tensors (layouts as mx_attention_forward).
    Returns O_lo, O_hi (q's shape) and LSE_lo, LSE_hi ([B, H, S] or [H, T])."""
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    O_lo, O_hi = np.zeros_like(q), np.zeros_like(q)
    shp = (q.shape[0], q.shape[2], q.shape[1]) if cu_seqlens is None else (q.shape[1], q.shape[0])
    L_lo, L_hi = np.zeros(shp), np.zeros(shp)
    ks, vs = dict(_heads(k, cu_seqlens)), dict(_heads(v, cu_seqlens))
    for key, qh in _heads(q, cu_seqlens):
        if qh.shape[0] == 0:
            continue
        b = forward_head_bounds(qh, ks[key], vs[key], sigma, causal, qk_fmt=qk_fmt)
        a, h = key
        if cu_seqlens is None:
            O_lo[a, :, h, :], O_hi[a, :, h, :] = b["O_lo"], b["O_hi"]
            L_lo[a, h, :], L_hi[a, h, :] = b["LSE_lo"], b["LSE_hi"]
        else:
            sl = slice(cu_seqlens[a], cu_seqlens[a + 1])
            O_lo[sl, h, :], O_hi[sl, h, :] = b["O_lo"], b["O_hi"]
            L_lo[h, sl], L_hi[h, sl] = b["LSE_lo"], b["LSE_hi"]
    return O_lo, O_hi, L_lo, L_hi


def mx_attention_backward_bounds(q, k, v, o, do, lse, sigma, causal, cu_seqlens=None, qk_fmt="e4m3"):
    """backward_bounds over whole tensors; returns {"dQ": (lo, hi), "dK": ..., "dV": ...} in the
    inputs' layout.  ``qk_fmt``: element format of Q and K."""
    q, k, v, o, do = (np.asarray(a, np.float64) for a in (q, k, v, o, do))
    lse = np.asarray(lse, np.float64)
    out = {n: (np.zeros_like(q), np.zeros_like(q)) for n in ("dQ", "dK", "dV")}
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
        b = backward_bounds(qh, K[key], V[key], Oh[key], DOh[key], lh, sigma, causal, qk_fmt=qk_fmt)
        for n in out:
            out[n][0][sl], out[n][1][sl] = b[n]
    return out
