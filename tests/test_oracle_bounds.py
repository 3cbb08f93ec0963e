"""Pins for the oracle's admissible-result bounds and for the backward's block layouts (CPU).

The attention oracle computes the plain definition, with every product of MX operands the
exact sum rounded once to fp32.  A matrix unit whose products differ from that by up to the
stated bound eps (oracle/gemm.py) can move P and dS codes across rounding boundaries, so the
parity tests accept any result inside forward_head_bounds / backward_bounds.  These bounds
are pinned here against things outside themselves:
  * with the slack switched off they collapse onto the plain oracle;
  * the plain oracle's own result lies inside them;
  * the plain oracle run with products perturbed by any delta in [-eps, eps] (random, and at
    the extremes +-eps) lands inside them -- the bounds hold what they claim to hold;
  * the instruction model (tests/hw/mfma_model.py, a measured characterisation of gfx950's
    block-scaled instruction) lands inside them on a workload with 50x outliers;
  * round_interval against brute-force quantization of sampled values;
  * tightness: plausible mistakes planted in the oracle (a 1% softmax-scale error, LSE in the
    wrong log base, D_i dropped from dS, a flipped sign, the causal diagonal hidden) fall outside.
Besides: the backward's online quantizations are pinned to their blockings ([News],
forward/backward and contributions paragraphs: dS in square [32 x 32] blocks, P for dV in
blocks of 32 queries per key) by a hand-derived closed form that every other blocking
violates, and the jagged scale offsets by literal values.
"""
import math

import numpy as np
import pytest

import synth
from hw import mfma_model as model
from oracle import attention as at
from oracle import gemm, mx


def _rand(shape, seed, outliers=0.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape)
    if outliers:
        x = np.where(rng.random(shape) < outliers, 50 * x, x)
    return x.astype(np.float32).astype(np.float64)


def _inside(x, lo, hi, slack=0.0):
    return bool(np.all((lo - slack <= x) & (x <= hi + slack)))


def _case(seed, L=96, D=64, outliers=0.0):
    q, k, v, do = (_rand((L, D), seed + i, outliers) for i in range(4))
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
def test_forward_bounds_collapse_onto_the_oracle(causal):
    q, k, v, _ = _case(1, L=100)
    f = at.forward_head(q, k, v, 0.125, causal)
    b = at.forward_head_bounds(q, k, v, 0.125, causal, mma=False, fp32=False)
    scale = np.max(np.abs(f["O"]))
    assert np.max(np.abs(b["O_lo"] - f["O"])) <= 1e-13 * scale
    assert np.max(np.abs(b["O_hi"] - f["O"])) <= 1e-13 * scale
    assert np.max(np.abs(b["LSE_lo"] - f["LSE"])) <= 1e-12 and np.max(np.abs(b["LSE_hi"] - f["LSE"])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_backward_bounds_collapse_onto_the_oracle(causal):
    q, k, v, do = _case(2, L=100)
    f = at.forward_head(q, k, v, 0.125, causal)
    o, lse = at.bf16(f["O"]), at.fl32(f["LSE"])
    g = at.backward_head(q, k, v, o, do, lse, 0.125, causal)
    b = at.backward_bounds(q, k, v, o, do, lse, 0.125, causal, mma=False, fp32=False)
    for n in ("dQ", "dK", "dV"):
        scale = np.max(np.abs(g[n]))
        assert np.max(np.abs(b[n][0] - g[n])) <= 1e-12 * scale, n
        assert np.max(np.abs(b[n][1] - g[n])) <= 1e-12 * scale, n


@pytest.mark.parametrize("outliers", [0.0, 0.01])
def test_exact_result_lies_inside_the_bounds(outliers):
    q, k, v, do = _case(3, L=128, outliers=outliers)
    f = at.forward_head(q, k, v, 0.125, True)
    b = at.forward_head_bounds(q, k, v, 0.125, True)
    assert _inside(f["O"], b["O_lo"], b["O_hi"]) and _inside(f["LSE"], b["LSE_lo"], b["LSE_hi"])
    o, lse = at.bf16(f["O"]), at.fl32(f["LSE"])
    g = at.backward_head(q, k, v, o, do, lse, 0.125, True)
    bb = at.backward_bounds(q, k, v, o, do, lse, 0.125, True)
    for n in ("dQ", "dK", "dV"):
        assert _inside(g[n], *bb[n]), n


def _eps_fwd(q, k):
    qv, qm = at._quantize_qk(q, "e4m3")
    kv, km = at._quantize_qk(k, "e4m3")
    return gemm.product_error_bound(qm, km)


def _eps_bwd(q, k, v, do):
    (_, qm), (_, km), (_, dm) = at._quantize_sq(q), at._quantize_sq(k), at._quantize_sq(do)
    _, vm = at._quantize_row(v)
    return gemm.product_error_bound(qm, km), gemm.product_error_bound(dm, vm)


@pytest.mark.parametrize("mode", ["random", "plus", "minus", "alternating"])
def test_bounds_hold_every_eps_close_product(mode):
    """Soundness: the plain oracle with every product moved by some delta, |delta| <= eps, stays
    inside the bounds (forward and backward; 1% outliers so that codes really move)."""
    rng = np.random.default_rng(4)
    q, k, v, do = _case(5, L=128, outliers=0.01)
    sig = 0.125

    def delta(eps):
        if mode == "random":
            return eps * rng.uniform(-1, 1, eps.shape)
        if mode == "plus":
            return eps
        if mode == "minus":
            return -eps
        return eps * np.where((np.arange(eps.shape[0])[:, None] + np.arange(eps.shape[1])) % 2, 1.0, -1.0)

    eps = _eps_fwd(q, k)
    b = at.forward_head_bounds(q, k, v, sig, True)
    fp = at.forward_head(q, k, v, sig, True, s_delta=delta(eps))
    assert _inside(fp["O"], b["O_lo"], b["O_hi"]) and _inside(fp["LSE"], b["LSE_lo"], b["LSE_hi"])
    f = at.forward_head(q, k, v, sig, True)
    o, lse = at.bf16(f["O"]), at.fl32(f["LSE"])
    eS, eP = _eps_bwd(q, k, v, do)
    bb = at.backward_bounds(q, k, v, o, do, lse, sig, True)
    gp = at.backward_head(q, k, v, o, do, lse, sig, True, s_delta=delta(eS), dp_delta=delta(eP))
    for n in ("dQ", "dK", "dV"):
        assert _inside(gp[n], *bb[n]), n


def test_instruction_model_lies_inside_the_bounds():
    """The small workload's outliers (0.1% of entries x50) on two heads, first 256 tokens: the
    forward and backward computed with the instruction model's S (and dP) stay inside the bounds
    (on the full workload they differ from the plain oracle by more than the comparison
    tolerances: O by up to ~100x 1e-3 max|O|, dQ by up to 8e-2 relative Frobenius)."""
    w = synth.workload("small")
    sig = 1 / math.sqrt(w.D)
    L = 256
    for h in (0, 3):
        q, k, v, do = (synth.tensor_np(w, t).double().numpy()[0, :L, h] for t in ("q", "k", "v", "do"))
        (qc, qk), (kc, kk) = mx.quantize_row32(q), mx.quantize_row32(k)
        qv, kv = mx.dequantize_row32(qc, qk), mx.dequantize_row32(kc, kk)
        s_hw = model.matmul_mfma(qv, mx.element_exponent_row32(qc, qk), kv, mx.element_exponent_row32(kc, kk))
        fm = at.forward_head(q, k, v, sig, True, s_delta=s_hw - qv @ kv.T)
        b = at.forward_head_bounds(q, k, v, sig, True)
        assert _inside(fm["O"], b["O_lo"], b["O_hi"]) and _inside(fm["LSE"], b["LSE_lo"], b["LSE_hi"])
        f = at.forward_head(q, k, v, sig, True)
        o, lse = at.bf16(f["O"]), at.fl32(f["LSE"])
        sq = [mx.quantize_sq32(x, 0) for x in (q, k, do)]
        (qv, qe), (kv, ke), (dv, de) = ((mx.dequantize_sq32(c, s, 0), mx.element_exponent_sq32(c, s, 0))
                                        for c, s in sq)
        vc, vk = mx.quantize_row32(v)
        vv, ve = mx.dequantize_row32(vc, vk), mx.element_exponent_row32(vc, vk)
        gm_ = at.backward_head(q, k, v, o, do, lse, sig, True,
                               s_delta=model.matmul_mfma(qv, qe, kv, ke) - qv @ kv.T,
                               dp_delta=model.matmul_mfma(dv, de, vv, ve) - dv @ vv.T)
        bb = at.backward_bounds(q, k, v, o, do, lse, sig, True)
        for n in ("dQ", "dK", "dV"):
            assert _inside(gm_[n], *bb[n]), (h, n)


@pytest.mark.parametrize("bq,bk", [(1, 32), (32, 1), (32, 32)])
def test_round_interval_holds_every_rounding(bq, bk):
    """lo == hi gives the plain MX rounding (blocks of bq x bk); otherwise any value between lo and
    hi, with the block amax it implies, rounds into [qlo, qhi] (brute force on sampled points)."""
    rng = np.random.default_rng(9)
    x = _rand((64, 64), 10) * np.exp2(rng.integers(-4, 4, (64, 1)))
    qlo, qhi, _ = mx.round_interval(x, x, bq, bk, floor_codes=(0,))
    ref = mx.dequantize_col32(*mx.quantize_col32(x, axis=1), axis=1) if (bq, bk) == (1, 32) else \
        mx.dequantize_col32(*mx.quantize_col32(x, axis=0), axis=0) if (bq, bk) == (32, 1) else \
        mx.dequantize_sq32(*mx.quantize_sq32(x, 0), 0)
    assert np.array_equal(qlo, ref) and np.array_equal(qhi, ref)
    w = np.abs(x) * 0.03
    lo, hi = x - w, x + w
    qlo, qhi, _ = mx.round_interval(lo, hi, bq, bk)
    for _ in range(20):
        y = lo + (hi - lo) * rng.random(x.shape)
        if (bq, bk) == (1, 32):
            qy = mx.dequantize_col32(*mx.quantize_col32(y, axis=1), axis=1)
        elif (bq, bk) == (32, 1):
            qy = mx.dequantize_col32(*mx.quantize_col32(y, axis=0), axis=0)
        else:
            qy = mx.dequantize_sq32(*mx.quantize_sq32(y, 0), 0)
        assert _inside(qy, qlo, qhi)


def test_round_interval_includes_both_scales_at_a_binade_edge():
    """A 32-element block whose amax interval [1.99, 2.01] straddles 2: scale codes 119 (2^-8) and
    120 (2^-7) are both admissible.  Normal elements keep E4M3's relative step under either scale;
    the two scales differ at the saturating top and in the subnormal range:
      * 1.875: 480 under 2^-8 saturates to 448 (1.75); 240 under 2^-7 is exact (1.875);
      * 3 2^-17: subnormal 3 2^-9 under 2^-8 (exact); 1.5 2^-9 under 2^-7 ties to 2 2^-9 (4 2^-17)."""
    lo = np.zeros((1, 32))
    hi = np.zeros((1, 32))
    lo[0, 0], hi[0, 0] = 1.99, 2.01
    lo[0, 1] = hi[0, 1] = 1.875
    lo[0, 2] = hi[0, 2] = 3 * 2.0 ** -17
    lo[0, 3] = hi[0, 3] = 1.25
    qlo, qhi, k = mx.round_interval(lo, hi, 1, 32)
    assert (qlo[0, 1], qhi[0, 1]) == (1.75, 1.875)
    assert (qlo[0, 2], qhi[0, 2]) == (3 * 2.0 ** -17, 4 * 2.0 ** -17)
    assert qlo[0, 3] == qhi[0, 3] == 1.25
    assert (qlo[0, 0], qhi[0, 0]) == (1.75, 2.0) and k[0, 0] == 120
    # with the amax pinned below 2, only code 119 remains
    hi[0, 0] = 1.995
    qlo, qhi, k = mx.round_interval(lo, hi, 1, 32)
    assert qlo[0, 1] == qhi[0, 1] == 1.75 and qlo[0, 2] == qhi[0, 2] == 3 * 2.0 ** -17 and k[0, 0] == 119


def test_backward_quantization_blockings_are_pinned():
    """Closed form that only the pages' blockings satisfy.  L = 32 queries and keys, causal,
    Q = 0 (so S' = 0 and p_ij = 2^-LSE_i log2 e), O = 0 (so D = 0), LSE_0 = 0 and LSE_i = 20 ln 2
    for i > 0: p_0j = 1 and p_ij ~ 2^-20.  dO row 0 = e_0, rows i > 0 = e_0 + e_1; V row 0 = e_0,
    row 1 = e_1, the rest 0.  Then dS is 1 at (0, 0) and ~2^-20 at (i, 0), (i, 1).
      * dS in one square [32 x 32] block: its amax is 1, every 2^-20 entry rounds to 0, so
        dQ_0 = sigma k^_0 and dQ_i = 0 for i > 0.  (Blocks of 32 keys per query keep rows i > 0;
        blocks of 32 queries per key keep column 1: both give dQ_i != 0.)
      * P for dV in blocks of 32 queries per key: key 0's block holds p_00 = 1, so
        dV_0 = dO^_0 = e_0; key j > 0 sees only p ~ 2^-20, kept as exactly 2^-20, so
        dV_j = (32 - j) 2^-20 (e_0 + e_1).  (Blocks of 32 keys per query would keep p_i0 in dV_0;
        square blocks would zero every dV_j, j > 0.)"""
    L, D, sig = 32, 64, 0.125
    q = np.zeros((L, D))
    k = _rand((L, D), 11)
    o = np.zeros((L, D))
    e0, e1 = np.eye(D)[0], np.eye(D)[1]
    do = np.tile(e0 + e1, (L, 1))
    do[0] = e0
    v = np.zeros((L, D))
    v[0], v[1] = e0, e1
    lse = np.full(L, float(np.float32(20 * math.log(2.0))))
    lse[0] = 0.0
    g = at.backward_head(q, k, v, o, do, lse, sig, True)
    kh = mx.dequantize_sq32(*mx.quantize_sq32(k, 0), 0)
    assert np.array_equal(g["dQ"][0], sig * kh[0])
    assert np.all(g["dQ"][1:] == 0)
    assert np.array_equal(g["dV"][0], e0)
    for j in range(1, L):
        assert np.array_equal(g["dV"][j], (L - j) * 2.0 ** -20 * (e0 + e1)), j
    assert np.all(g["dK"] == 0)


def test_padded_offsets_literal_values():
    """Scale rows of a jagged batch start at the prefix sum of each length rounded up to 128
    ([News], contributions paragraph: 128-aligned scale placement, packed payload)."""
    assert mx.padded_offsets([5, 128, 33, 200, 0, 64]).tolist() == [0, 128, 256, 384, 640, 640, 768]
    assert mx.padded_offsets([129]).tolist() == [0, 256]
    assert mx.padded_offsets([]).tolist() == [0]
    assert mx.padded_offsets([0, 0, 1]).tolist() == [0, 0, 0, 128]


def _outside_share(x, lo, hi):
    return float(np.mean((x < lo) | (x > hi)))


def test_bounds_catch_planted_mistakes():
    """Tightness: the admissible intervals are narrow enough that plausible kernel mistakes, planted
    here in the oracle on the CPU, land outside them -- a softmax scale off by 1% (a wrong c), the
    LSE left in log2 units, the D_i term dropped from dS (dS = p dP), dO's sign flipped in dP, and a
    causal mask that also hides the diagonal (rows shifted by one key)."""
    q, k, v, do = _case(7, L=128)
    sig = 0.125
    b = at.forward_head_bounds(q, k, v, sig, True)
    f = at.forward_head(q, k, v, sig, True)
    assert _inside(f["O"], b["O_lo"], b["O_hi"])
    wrong_c = at.forward_head(q, k, v, sig * 1.01, True)
    assert _outside_share(wrong_c["O"], b["O_lo"], b["O_hi"]) > 0.05
    assert _outside_share(f["LSE"] / math.log(2), b["LSE_lo"], b["LSE_hi"]) > 0.9
    # diagonal hidden too: row i sees keys < i, i.e. the causal result of keys shifted down by one
    k_shift, v_shift = np.roll(k, 1, axis=0), np.roll(v, 1, axis=0)
    no_diag = at.forward_head(q, k_shift, v_shift, sig, True)
    assert _outside_share(no_diag["O"][1:], b["O_lo"][1:], b["O_hi"][1:]) > 0.5
    o, lse = at.bf16(f["O"]), at.fl32(f["LSE"])
    bb = at.backward_bounds(q, k, v, o, do, lse, sig, True)
    no_d = at.backward_head(q, k, v, np.zeros_like(o), do, lse, sig, True)   # D_i = 0: dS = p dP
    for n in ("dQ", "dK"):
        assert _outside_share(no_d[n], *bb[n]) > 0.05, n
    flipped = at.backward_head(q, k, v, o, -do, lse, sig, True)              # every gradient negated
    for n in ("dQ", "dK", "dV"):
        assert _outside_share(flipped[n], *bb[n]) > 0.5, n
