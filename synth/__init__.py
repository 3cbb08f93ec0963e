"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This module only draws random numbers and lays them out in the shapes the
attention workloads use.  It holds none of the MX quantization or attention
arithmetic, so neither side of a parity test can borrow the other's maths
through it.

Generator: counter-based SplitMix64 (Steele, Lea and Flood, "Fast Splittable
Pseudorandom Number Generators", OOPSLA 2014).  Draw ``n`` of a stream is
``mix64(key + (n + 1) * GAMMA)`` with ``key = mix64(seed * 2**16 + stream)``,
so any element of any tensor can be produced on its own, on the CPU (numpy
uint64) or on a GPU (torch int64, same bits).  Normals use the cosine branch of
Box-Muller on draws ``2n`` and ``2n + 1`` in float64, then round to float32 and,
for bf16 inputs, round the float32 value to bf16 (round-to-nearest-even).

Streams: Q=0, K=1, V=2, dO=3, outlier mask=4, per-head scales=5,
sequence lengths=6, (batch, head) sample=7.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB
MASK64 = (1 << 64) - 1

STREAM_Q, STREAM_K, STREAM_V, STREAM_DO = 0, 1, 2, 3
STREAM_OUTLIER, STREAM_HEADSCALE, STREAM_SEQLEN, STREAM_SAMPLE = 4, 5, 6, 7
TENSOR_STREAMS = {"q": STREAM_Q, "k": STREAM_K, "v": STREAM_V, "do": STREAM_DO}


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int) -> int:
    return _mix64_int(seed * (1 << 16) + stream)


# ---------------------------------------------------------------- numpy (CPU)
def _mix64_np(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
    return z ^ (z >> np.uint64(31))


def u64_np(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(stream_key(seed, stream)) + (idx + np.uint64(1)) * np.uint64(GAMMA)
    return _mix64_np(z)


def uniform_np(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """Uniform in the open interval (0, 1), float64, 53 random bits."""
    u = u64_np(seed, stream, idx) >> np.uint64(11)
    return (u.astype(np.float64) + 0.5) * (2.0 ** -53)


def normal_np(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    idx = np.asarray(idx, dtype=np.uint64)
    u1 = uniform_np(seed, stream, idx * np.uint64(2))
    u2 = uniform_np(seed, stream, idx * np.uint64(2) + np.uint64(1))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


# ------------------------------------------------------------ torch (any dev)
def _signed(c: int) -> int:
    return c - (1 << 64) if c >= (1 << 63) else c


def _lsr(z, k: int):
    """Logical right shift of int64 bit patterns."""
    import torch
    return torch.bitwise_and(torch.bitwise_right_shift(z, k), (1 << (64 - k)) - 1)


def _mix64_torch(z):
    z = torch_xor(z, _lsr(z, 30)) * _signed(MIX1)
    z = torch_xor(z, _lsr(z, 27)) * _signed(MIX2)
    return torch_xor(z, _lsr(z, 31))


def torch_xor(a, b):
    import torch
    return torch.bitwise_xor(a, b)


def uniform_torch(seed: int, stream: int, idx):
    z = _signed(stream_key(seed, stream)) + (idx + 1) * _signed(GAMMA)
    u = _lsr(_mix64_torch(z), 11)
    import torch
    return (u.to(torch.float64) + 0.5) * (2.0 ** -53)


def normal_torch(seed: int, stream: int, idx):
    import torch
    u1 = uniform_torch(seed, stream, idx * 2)
    u2 = uniform_torch(seed, stream, idx * 2 + 1)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)


# --------------------------------------------------------------- workloads
@dataclass
class Workload:
    """One seeded synthetic attention problem.

    Fixed-length problems use [B, S, H, D] tensors; varlen problems pack
    sequences as [T, H, D] with ``cu_seqlens`` (int32, nseq + 1).
    """
    name: str
    seed: int
    B: int
    S: int
    H: int
    D: int
    causal: bool
    dtype: str = "bf16"            # input/output element type: "bf16" or "fp32"
    outlier_rate: float = 0.0      # Bernoulli rate of entries multiplied by outlier_mult
    outlier_mult: float = 50.0
    head_scale: bool = False       # per-(tensor, head) scale 10**U(-1, 1)
    grid: bool = False             # values +-(1 + m/8), m = 0..7, instead of normals
    seqlens: list = field(default_factory=list)  # varlen lengths (empty = fixed)

    @property
    def varlen(self) -> bool:
        return bool(self.seqlens)

    @property
    def total_tokens(self) -> int:
        return sum(self.seqlens) if self.varlen else self.B * self.S

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def numel(self) -> int:
        return self.total_tokens * self.H * self.D

    def shape(self):
        return (self.total_tokens, self.H, self.D) if self.varlen else (self.B, self.S, self.H, self.D)


def draw_seqlens(seed: int, nseq: int, lo: int, hi: int) -> list:
    """Integer lengths uniform on [lo, hi] inclusive."""
    u = uniform_np(seed, STREAM_SEQLEN, np.arange(nseq))
    return [int(lo + math.floor(x * (hi - lo + 1))) for x in u]


def draw_sample_pairs(seed: int, B: int, H: int, n: int) -> list:
    """n distinct (batch, head) pairs, drawn without replacement."""
    order = np.argsort(uniform_np(seed, STREAM_SAMPLE, np.arange(B * H)), kind="stable")
    return [(int(i) // H, int(i) % H) for i in order[:n]]


def workload(name: str) -> Workload:
    """The named synthetic workloads (shapes and value recipes)."""
    if name == "tiny":       # B1 H1 S128 D64, non-causal, fp32 in and out
        return Workload(name, 0, 1, 128, 1, 64, causal=False, dtype="fp32")
    if name == "small":      # B2 H8 S1024 D128 causal, 0.1% outliers x50
        return Workload(name, 1, 2, 1024, 8, 128, causal=True, outlier_rate=1e-3)
    if name == "llm":        # B8 H32 S8192 D128 causal
        return Workload(name, 2, 8, 8192, 32, 128, causal=True)
    if name == "long":       # B4 H16 S4096 D128 causal, per-head log-uniform scales
        return Workload(name, 3, 4, 4096, 16, 128, causal=True, head_scale=True)
    if name == "grid":       # B2 H4 S1000 D128 causal, values +-(1 + m/8): every block scale equal and
        # every product of two elements in two adjacent binades, so a matrix unit adds them exactly
        return Workload(name, 5, 2, 1000, 4, 128, causal=True, grid=True)
    if name == "varlen":     # 16 sequences, lengths U{256..8192}, H16 D128 causal
        seed = 4
        return Workload(name, seed, 16, 0, 16, 128, causal=True, seqlens=draw_seqlens(seed, 16, 256, 8192))
    raise KeyError(name)


def _tensor_id(which: str) -> int:
    return TENSOR_STREAMS[which]


def head_scales_np(w: Workload, which: str) -> np.ndarray:
    if not w.head_scale:
        return np.ones(w.H)
    u = uniform_np(w.seed, STREAM_HEADSCALE, _tensor_id(which) * w.H + np.arange(w.H))
    return 10.0 ** (2.0 * u - 1.0)


def _finish_np(w: Workload, which: str, z: np.ndarray, idx: np.ndarray, head: np.ndarray):
    """Apply outliers and head scales in float64, round to float32 (and bf16)."""
    import torch
    if w.outlier_rate > 0:
        u = uniform_np(w.seed, STREAM_OUTLIER, np.uint64(_tensor_id(which) * w.numel()) + idx.astype(np.uint64))
        z = np.where(u < w.outlier_rate, z * w.outlier_mult, z)
    if w.head_scale:
        z = z * head_scales_np(w, which)[head]
    x32 = torch.from_numpy(z.astype(np.float32))
    return x32 if w.dtype == "fp32" else x32.to(torch.bfloat16)


def grid_np(seed: int, stream: int, idx: np.ndarray) -> np.ndarray:
    """+-(1 + m/8): u = uniform draw, j = floor(16 u); sign - for j >= 8, m = j mod 8."""
    j = np.floor(uniform_np(seed, stream, idx) * 16.0)
    return np.where(j >= 8, -1.0, 1.0) * (1.0 + np.mod(j, 8.0) / 8.0)


def grid_torch(seed: int, stream: int, idx):
    import torch
    j = torch.floor(uniform_torch(seed, stream, idx) * 16.0)
    return torch.where(j >= 8, -1.0, 1.0).to(torch.float64) * (1.0 + torch.remainder(j, 8.0) / 8.0)


def _draw_np(w: Workload, which: str, idx: np.ndarray) -> np.ndarray:
    return (grid_np if w.grid else normal_np)(w.seed, _tensor_id(which), idx)


def tensor_np(w: Workload, which: str):
    """The whole input tensor on the CPU (torch, float32 or bfloat16)."""
    n = w.numel()
    idx = np.arange(n, dtype=np.uint64)
    z = _draw_np(w, which, idx)
    head = (np.arange(n) // w.D) % w.H
    return _finish_np(w, which, z, idx, head).reshape(w.shape())


def head_slice_np(w: Workload, which: str, b: int, h: int):
    """One (batch, head) slice [S, D] of a fixed-length tensor, on the CPU."""
    assert not w.varlen
    s = np.arange(w.S, dtype=np.uint64)[:, None]
    d = np.arange(w.D, dtype=np.uint64)[None, :]
    idx = ((np.uint64(b) * np.uint64(w.S) + s) * np.uint64(w.H) + np.uint64(h)) * np.uint64(w.D) + d
    z = _draw_np(w, which, idx)
    return _finish_np(w, which, z, idx, np.full(idx.shape, h))


def token_slice_np(w: Workload, which: str, t0: int, t1: int, h: int):
    """Tokens t0..t1-1 (flat token index: b * S + s, or the packed position) of head h, [t1 - t0, D],
    on the CPU; the same bits as the whole tensor's slice."""
    t = np.arange(t0, t1, dtype=np.uint64)[:, None]
    d = np.arange(w.D, dtype=np.uint64)[None, :]
    idx = (t * np.uint64(w.H) + np.uint64(h)) * np.uint64(w.D) + d
    z = _draw_np(w, which, idx)
    return _finish_np(w, which, z, idx, np.full(idx.shape, h))


def tensor_torch(w: Workload, which: str, device, chunk: int = 1 << 26):
    """The whole input tensor generated on ``device`` with the same bits as tensor_np."""
    import torch
    n = w.numel()
    out = torch.empty(n, dtype=torch.float32 if w.dtype == "fp32" else torch.bfloat16, device=device)
    hs = torch.tensor(head_scales_np(w, which), dtype=torch.float64, device=device)
    for s0 in range(0, n, chunk):
        idx = torch.arange(s0, min(n, s0 + chunk), dtype=torch.int64, device=device)
        z = (grid_torch if w.grid else normal_torch)(w.seed, _tensor_id(which), idx)
        if w.outlier_rate > 0:
            u = uniform_torch(w.seed, STREAM_OUTLIER, idx + _tensor_id(which) * n)
            z = torch.where(u < w.outlier_rate, z * w.outlier_mult, z)
        if w.head_scale:
            z = z * hs[(idx // w.D) % w.H]
        out[s0:s0 + idx.numel()] = z.to(torch.float32).to(out.dtype)
    return out.reshape(w.shape())
