"""Pins for the oracle's MX attention (CPU only).

The oracle is tied to things outside itself: float64 textbook attention
(with quantization and fp32 rounding switched off it must agree to 1e-12),
central finite differences of that textbook forward, closed forms of the
integer-frame softmax, an independent online (tiled) emulation of the forward
that must reproduce the oracle's P-hat codes bit for bit, inputs built to be
exactly representable in one MX layout (so the layout each operand uses is
pinned), and the cosine >= 0.99 accuracy bar against float64 attention.
"""
import math

import numpy as np
import pytest

import synth
from oracle import attention as at
from oracle import mx


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _cos(a, b):
    a, b = np.ravel(a), np.ravel(b)
    return float(a @ b / np.linalg.norm(a) / np.linalg.norm(b))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("L,D", [(1, 64), (37, 64), (100, 128)])
def test_forward_skeleton_equals_textbook(L, D, causal):
    q, k, v = (_rand((L, D), s) for s in (1, 2, 3))
    sigma = 1 / math.sqrt(D)
    r = at.forward_head(q, k, v, sigma, causal, quantize=False, exact=True)
    O, lse = at.attention_fp64(q, k, v, sigma, causal)
    assert np.max(np.abs(r["O"] - O)) <= 1e-12 * max(1, np.max(np.abs(O)))
    assert np.max(np.abs(r["LSE"] - lse)) <= 1e-12 * max(1, np.max(np.abs(lse)))


@pytest.mark.parametrize("causal", [False, True])
def test_backward_skeleton_equals_textbook(causal):
    L, D = 45, 64
    q, k, v, do = (_rand((L, D), s) for s in (4, 5, 6, 7))
    sigma = 0.2
    O, lse = at.attention_fp64(q, k, v, sigma, causal)
    g = at.backward_head(q, k, v, O, do, lse, sigma, causal, quantize=False, exact=True)
    ref = at.attention_fp64_backward(q, k, v, do, sigma, causal)
    for a, b in zip((g["dQ"], g["dK"], g["dV"]), ref):
        assert np.max(np.abs(a - b)) <= 1e-12 * max(1, np.max(np.abs(b)))


def test_textbook_backward_matches_finite_differences():
    L, D = 9, 32
    q, k, v, do = (_rand((L, D), s) for s in (8, 9, 10, 11))
    sigma, causal = 0.3, True
    dq, dk, dv = at.attention_fp64_backward(q, k, v, do, sigma, causal)
    h = 1e-6
    rng = np.random.default_rng(0)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            i, j = rng.integers(L), rng.integers(D)
            xp, xm = x.copy(), x.copy()
            xp[i, j] += h
            xm[i, j] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            fp = np.sum(at.attention_fp64(args["q"], args["k"], args["v"], sigma, causal)[0] * do)
            args[name] = xm
            fm = np.sum(at.attention_fp64(args["q"], args["k"], args["v"], sigma, causal)[0] * do)
            assert abs((fp - fm) / (2 * h) - g[i, j]) <= 1e-6 * max(1, abs(g[i, j]))


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    L, D = 80, 64
    k, v = _rand((L, D), 12), _rand((L, D), 13)
    r = at.forward_head(np.zeros((L, D)), k, v, 0.125, causal)
    vh = mx.dequantize_col32(*mx.quantize_col32(v, axis=0), axis=0)
    n = np.arange(1, L + 1) if causal else np.full(L, L)
    ref = np.cumsum(vh, axis=0) / n[:, None] if causal else np.tile(vh.mean(0), (L, 1))
    assert np.allclose(r["O"], ref, rtol=0, atol=1e-14)
    assert np.allclose(r["LSE"], np.log(n), rtol=0, atol=1e-14)
    assert np.all(r["M"] == 0)


def test_causal_first_row_closed_form():
    L, D = 40, 128
    q, k, v = (_rand((L, D), s) for s in (14, 15, 16))
    sigma = 1 / math.sqrt(D)
    r = at.forward_head(q, k, v, sigma, True)
    qh = mx.dequantize_row32(*mx.quantize_row32(q))
    kh = mx.dequantize_row32(*mx.quantize_row32(k))
    s00 = float(np.float32(qh[0] @ kh[0]))
    p = np.float32(2.0 ** np.float32(s00 * at.log2_scale(sigma) - r["M"][0]))
    phat = mx.dequantize_blocks(*mx.quantize_blocks(np.array([[float(p)] + [0.0] * 31])))[0, 0]
    vh = mx.dequantize_col32(*mx.quantize_col32(v, axis=0), axis=0)
    assert np.allclose(r["O"][0], phat / p * vh[0], rtol=1e-15, atol=0)
    assert abs(r["LSE"][0] - sigma * s00) <= 1e-6 * max(1, abs(sigma * s00))


def test_power_of_two_value_scaling_is_exact():
    L, D = 64, 64
    q, k, v = (_rand((L, D), s) for s in (17, 18, 19))
    a = at.forward_head(q, k, v, 0.125, True)["O"]
    b = at.forward_head(q, k, v * 2.0 ** 5, 0.125, True)["O"]
    assert np.array_equal(b, a * 2.0 ** 5)


def test_one_hot_row_reading_discriminator():
    """A single dominant key: the integer frame gives O = (MX(p)/p) v-hat, not v-hat."""
    L, D = 32, 64
    k = _rand((L, D), 20) * 0.01
    v = _rand((L, D), 21)
    q = np.zeros((L, D))
    q[:] = 0.01 * _rand((L, D), 22)
    k[7] = 1.0
    q[31] = 40.0                       # row 31 attends almost only to key 7
    r = at.forward_head(q, k, v, 1.0, True)
    p7 = r["l"][31]                    # all other p underflow to ~0
    phat = mx.dequantize_blocks(*mx.quantize_blocks(np.array([[p7] + [0.0] * 31])))[0, 0]
    vh = mx.dequantize_col32(*mx.quantize_col32(v, axis=0), axis=0)
    assert np.allclose(r["O"][31], phat / p7 * vh[7], rtol=1e-9, atol=1e-300)


def test_softmax_rows_sum_to_one():
    L, D = 128, 64
    q, k, v = (_rand((L, D), s) * 2 for s in (23, 24, 25))
    for causal in (False, True):
        r = at.forward_head(q, k, v, 0.125, causal)
        vis = at.visible(L, L, causal)
        S = np.where(vis, r["S"], -np.inf)
        c = at.log2_scale(0.125)
        p = np.where(vis, at.fl32(np.exp2(at.fl32(S * c - r["M"][:, None]))), 0)
        assert np.allclose(p.sum(1) / r["l"], 1, rtol=1e-12, atol=0)
        ph = mx.dequantize_col32(r["P_codes"], r["P_scales"], axis=1)
        assert np.all(np.abs(ph.sum(1) / r["l"] - 1) <= 1 / 8)


def _online_forward(q, k, v, sigma, causal, Bc, lazy):
    """Tiled forward with a running integer frame (exact float64 arguments)."""
    L, D = q.shape
    qh = mx.dequantize_row32(*mx.quantize_row32(q))
    kh = mx.dequantize_row32(*mx.quantize_row32(k))
    vh = mx.dequantize_col32(*mx.quantize_col32(v, axis=0), axis=0)
    c = sigma * math.log2(math.e)
    M = np.full(L, -np.inf)
    lsum = np.zeros(L)
    acc = np.zeros((L, D))
    codes = np.zeros((L, L), np.uint8)
    scl = np.zeros((L, (L + 31) // 32), np.int64)
    for j0 in range(0, L, Bc):
        j1 = min(L, j0 + Bc)
        t = (qh @ kh[j0:j1].T) * c
        vis = at.visible(L, L, causal)[:, j0:j1]
        tmax = np.max(np.where(vis, t, -np.inf), axis=1)
        need = np.ceil(tmax)
        Mn = np.where(lazy & (need <= M + 4), M, np.maximum(M, need))
        fac = np.where(np.isfinite(M), np.exp2(M - Mn), 0.0)
        acc *= fac[:, None]
        lsum *= fac
        M = np.where(np.isfinite(Mn), Mn, M)
        p = np.where(vis, np.exp2(t - M[:, None]), 0.0)
        lsum += p.sum(1)
        pc, pk = mx.quantize_col32(p, axis=1)
        acc += mx.dequantize_col32(pc, pk, axis=1) @ vh[j0:j1]
        codes[:, j0:j1] = pc
        # frame-free scale exponent of each non-empty block (empty blocks keep code 0)
        scl[:, j0 // 32:(j1 + 31) // 32] = np.where(pk > 0, pk.astype(np.int64) + M[:, None].astype(np.int64), 0)
    return acc / lsum[:, None], codes, scl


@pytest.mark.parametrize("Bc", [32, 64, 128])
@pytest.mark.parametrize("lazy", [False, True])
def test_online_tiling_reproduces_two_pass_codes(Bc, lazy):
    L, D = 192, 64
    q, k, v = (_rand((L, D), s) * 1.5 for s in (26, 27, 28))
    sigma = 1 / 8
    ref = at.forward_head(q, k, v, sigma, True, exact=True)
    O, codes, scl = _online_forward(q, k, v, sigma, True, Bc, lazy)
    assert np.array_equal(codes, ref["P_codes"])
    rk = ref["P_scales"].astype(np.int64)
    assert np.array_equal(scl, np.where(rk > 0, rk + ref["M"][:, None].astype(np.int64), 0))
    assert np.max(np.abs(O - ref["O"])) <= 1e-12 * np.max(np.abs(ref["O"]))


def _representable(rng, shape, block_axes):
    """Values that one MX layout holds exactly: per block, E4M3 codes times a
    block scale, with one element of each block in the top binade."""
    x = mx.e4m3_decode(rng.integers(0x20, 0x7F, size=shape)) * rng.choice([-1, 1], size=shape)
    return x


def test_forward_operand_layouts_are_pinned():
    """Q, K exactly representable in ROW32 (blocks along D); V exactly
    representable in COL32 (blocks along keys).  Then S must be fl32(Q K^T)
    exactly, and with Q = 0 the output is the exact column mean of V."""
    rng = np.random.default_rng(30)
    L, D = 64, 64
    def row_exact(shape):
        x = mx.e4m3_decode(rng.integers(0x30, 0x7F, size=shape))
        x[..., ::32] = 320.0 * np.sign(rng.standard_normal(x[..., ::32].shape))  # a top-binade element per block
        return x * np.exp2(rng.integers(-12, 6, size=shape[:-1] + (1,)))
    q, k = row_exact((L, D)), row_exact((L, D))
    r = at.forward_head(q, k, _rand((L, D), 31), 0.1, False)
    assert np.array_equal(r["S"], at.fl32(q @ k.T))
    # V: each 32-key block of each column has its own power-of-two scale
    v = mx.e4m3_decode(rng.integers(0x30, 0x7F, size=(L, D)))
    v[::32, :] = 320.0
    v = v * np.exp2(np.repeat(rng.integers(-20, 20, size=(L // 32, D)), 32, axis=0))
    r = at.forward_head(np.zeros((L, D)), k, v, 0.1, False)
    assert np.allclose(r["O"], np.tile(v.mean(0), (L, 1)), rtol=1e-15, atol=0)
    # and V quantized along D would not be exact for this input
    assert not np.array_equal(mx.dequantize_row32(*mx.quantize_row32(v)), v)


def test_backward_operand_layouts_are_pinned():
    """Q, K, dO exactly representable in square [32, 32] blocks and V in
    ROW32: S' and dP must then be fl32 of the exact products."""
    rng = np.random.default_rng(32)
    L, D = 64, 64
    def sq_exact():
        x = mx.e4m3_decode(rng.integers(0x30, 0x7F, size=(L, D)))
        x[::32, ::32] = 320.0
        return x * np.exp2(np.repeat(np.repeat(rng.integers(-12, -6, size=(L // 32, D // 32)), 32, 0), 32, 1))
    q, k, do = sq_exact(), sq_exact(), sq_exact()
    v = mx.e4m3_decode(rng.integers(0x30, 0x7F, size=(L, D)))
    v[:, ::32] = 320.0
    v = v * np.exp2(rng.integers(-8, 8, size=(L, 1)))
    O, lse = at.attention_fp64(q, k, v, 0.05, True)
    g = at.backward_head(q, k, v, O, do, lse, 0.05, True)
    assert np.array_equal(g["S"], at.fl32(q @ k.T))
    assert np.array_equal(g["dP"], at.fl32(do @ v.T))
    assert np.array_equal(g["D"], at.fl32(np.sum(do * O, axis=1)))


@pytest.mark.parametrize("L,D,causal", [(128, 64, False), (128, 64, True), (256, 128, True), (200, 128, False)])
def test_accuracy_against_float64_attention(L, D, causal):
    q, k, v, do = (_rand((L, D), s) for s in (40, 41, 42, 43))
    sigma = 1 / math.sqrt(D)
    r = at.forward_head(q, k, v, sigma, causal)
    O, lse = at.attention_fp64(q, k, v, sigma, causal)
    assert _cos(r["O"], O) >= 0.99
    g = at.backward_head(q, k, v, r["O"], do, r["LSE"], sigma, causal)
    for a, b in zip((g["dQ"], g["dK"], g["dV"]), at.attention_fp64_backward(q, k, v, do, sigma, causal)):
        assert _cos(a, b) >= 0.99


def test_tiny_workload_accuracy():
    w = synth.workload("tiny")
    q, k, v = (synth.tensor_np(w, t).double().numpy()[0, :, 0, :] for t in ("q", "k", "v"))
    r = at.forward_head(q, k, v, 1 / 8, False)
    O, _ = at.attention_fp64(q, k, v, 1 / 8, False)
    assert _cos(r["O"], O) >= 0.99


def test_varlen_forward_equals_per_sequence():
    L = [40, 1, 97]
    cu = np.concatenate([[0], np.cumsum(L)])
    H, D = 2, 64
    q, k, v = (_rand((cu[-1], H, D), s) for s in (50, 51, 52))
    O, LSE = at.mx_attention_forward(q, k, v, 0.125, True, cu_seqlens=cu)
    for s in range(len(L)):
        for h in range(H):
            r = at.forward_head(q[cu[s]:cu[s + 1], h], k[cu[s]:cu[s + 1], h], v[cu[s]:cu[s + 1], h], 0.125, True)
            assert np.array_equal(O[cu[s]:cu[s + 1], h], r["O"])
            assert np.array_equal(LSE[h, cu[s]:cu[s + 1]], r["LSE"])


@pytest.mark.parametrize("causal", [True, False])
def test_backward_blocks_equal_the_full_backward(causal):
    """The block-subset backward (used to check full-size kernels on sampled blocks) returns
    exactly the rows of the full quantized backward, including a short tail block."""
    rng = np.random.default_rng(21)
    L, D, sigma = 150, 64, 0.125
    q, k, v, do = (rng.standard_normal((L, D)).astype(np.float32).astype(np.float64) for _ in range(4))
    f = at.forward_head(q, k, v, sigma, causal)
    o, lse = f["O"].astype(np.float32).astype(np.float64), f["LSE"].astype(np.float32).astype(np.float64)
    full = at.backward_head(q, k, v, o, do, lse, sigma, causal)
    blocks = [0, 2, 4]   # block 4 holds rows 128..149
    part = at.backward_head_blocks(q, k, v, o, do, lse, sigma, causal, q_blocks=blocks, k_blocks=blocks)
    for b in blocks:
        rows = slice(32 * b, min(L, 32 * b + 32))
        assert np.array_equal(part["dQ"][b], full["dQ"][rows])
        assert np.array_equal(part["dK"][b], full["dK"][rows])
        assert np.array_equal(part["dV"][b], full["dV"][rows])
