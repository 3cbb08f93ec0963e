"""Pins of the oracle's BF16 attention baseline (quantization off, P rounded to
bfloat16 before P V), independent of any kernel:
  * the rounding helper against torch's fp32 -> bfloat16 conversion and hand
    cases (ties to even, carries into the exponent);
  * when every p is a power of two, rounding changes nothing: O equals the
    quantization-off path bit for bit;
  * otherwise each O element moves by at most 2^-8 sum_j p_j |v_jd| / l_i (the
    unit roundoff of bfloat16 applied to every P entry), and it does move."""
import math

import numpy as np
import pytest
import torch

from oracle import attention as at


def test_bf16_rounding_matches_torch_and_hand_cases():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    # exact ties: 16 low bits = 0x8000 with odd and even kept parts
    u = rng.integers(0, 2**31, 2000, dtype=np.uint64).astype(np.uint32) & np.uint32(0x7F7F0000)
    ties = (u | np.uint32(0x8000)).view(np.float32)
    for arr in (x, ties):
        ref = torch.from_numpy(arr.copy()).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.array_equal(at.bf16(arr), ref)
    one = 1.0
    assert at.bf16(one + 2.0**-8) == 1.0                      # tie, kept part even: down
    assert at.bf16(1.0 + 3 * 2.0**-8) == 1.0 + 2.0**-6         # tie, kept part odd: up
    assert at.bf16(1.0 + 2.0**-8 + 2.0**-20) == 1.0 + 2.0**-7  # above the tie: up
    assert at.bf16(2.0 - 2.0**-23) == 2.0                       # carry into the exponent
    assert at.bf16(-1.5) == -1.5 and at.bf16(0.0) == 0.0


def test_power_of_two_p_is_unchanged_by_bf16_rounding():
    # sigma = fl32(ln 2) gives c = 1 exactly; integer logits make every p = 2^integer
    sigma = float(np.float32(math.log(2)))
    assert at.log2_scale(sigma) == 1.0
    rng = np.random.default_rng(1)
    L, D = 96, 64
    q = rng.integers(-2, 3, (L, D)).astype(np.float64)
    k = rng.integers(-2, 3, (L, D)).astype(np.float64) / 8.0   # logits are multiples of 1/8 ...
    k = np.round(k)                                             # ... made integers
    v = rng.standard_normal((L, D)).astype(np.float32).astype(np.float64)
    for causal in (False, True):
        a = at.forward_head(q, k, v, sigma, causal, quantize=False)
        b = at.forward_head(q, k, v, sigma, causal, quantize=False, p_round="bf16")
        assert np.array_equal(a["O"], b["O"]) and np.array_equal(a["LSE"], b["LSE"])


@pytest.mark.parametrize("causal", [False, True])
def test_bf16_p_error_bound(causal):
    rng = np.random.default_rng(2)
    L, D, sigma = 160, 64, 1 / 8
    q, k, v = (rng.standard_normal((L, D)).astype(np.float32).astype(np.float64) for _ in range(3))
    a = at.forward_head(q, k, v, sigma, causal, quantize=False)
    b = at.forward_head(q, k, v, sigma, causal, quantize=False, p_round="bf16")
    vis = at.visible(L, L, causal)
    c = at.log2_scale(sigma)
    p = np.where(vis, np.exp2(a["S"] * c - a["M"][:, None]), 0.0)
    bound = 2.0**-8 * (p @ np.abs(v)) / a["l"][:, None] * (1 + 1e-6)
    diff = np.abs(b["O"] - a["O"])
    assert np.all(diff <= bound)
    assert np.max(diff) > 0 and np.array_equal(a["LSE"], b["LSE"])


def test_backward_bf16_rounding_is_exact_on_representable_p_and_ds():
    # c = 1, lse = 0, o = 0 (so D = 0) and integer q, k, v, dO: p = 2^S and dS = p dP are bf16-exact
    sigma = float(np.float32(math.log(2)))
    rng = np.random.default_rng(3)
    L, D = 64, 32
    q = rng.integers(-1, 2, (L, D)).astype(np.float64)
    k = rng.integers(-1, 2, (L, D)).astype(np.float64)
    v = rng.integers(-2, 3, (L, D)).astype(np.float64)
    do = rng.integers(-2, 3, (L, D)).astype(np.float64)
    o, lse = np.zeros((L, D)), np.zeros(L)
    for causal in (False, True):
        a = at.backward_head(q, k, v, o, do, lse, sigma, causal, quantize=False)
        b = at.backward_head(q, k, v, o, do, lse, sigma, causal, quantize=False, p_round="bf16")
        assert np.max(np.abs(a["dS"])) > 1                      # not a trivial case
        for g in ("dQ", "dK", "dV"):
            assert np.array_equal(a[g], b[g]), g


@pytest.mark.parametrize("causal", [False, True])
def test_backward_bf16_error_bounds(causal):
    rng = np.random.default_rng(4)
    L, D, sigma = 96, 64, 1 / 8
    q, k, v, do = (rng.standard_normal((L, D)).astype(np.float32).astype(np.float64) for _ in range(4))
    f = at.forward_head(q, k, v, sigma, causal, quantize=False)
    o, lse = f["O"].astype(np.float32).astype(np.float64), f["LSE"].astype(np.float32).astype(np.float64)
    a = at.backward_head(q, k, v, o, do, lse, sigma, causal, quantize=False)
    b = at.backward_head(q, k, v, o, do, lse, sigma, causal, quantize=False, p_round="bf16")
    u = 2.0**-8 * (1 + 1e-6)
    assert np.all(np.abs(b["dV"] - a["dV"]) <= u * (np.abs(a["p"]).T @ np.abs(do)))
    assert np.all(np.abs(b["dK"] - a["dK"]) <= u * sigma * (np.abs(a["dS"]).T @ np.abs(q)))
    assert np.all(np.abs(b["dQ"] - a["dQ"]) <= u * sigma * (np.abs(a["dS"]) @ np.abs(k)))
    for g in ("dQ", "dK", "dV"):
        assert np.max(np.abs(b[g] - a[g])) > 0, g
