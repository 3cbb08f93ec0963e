"""Benchmark of the MXFP8 attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step = MX quantization of Q, K, V, dO in every layout the forward and
backward consume, the fused forward, and the fused backward, on the
synthetic LLM-shaped workload (B8 H32 S8192 D128, causal, bf16 N(0,1)
inputs already resident in HBM).  Prints one JSON line.  Kernel durations
come from HIP events recorded on the stream the kernels run on.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MXFP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 / MXFP8 MFMA peak
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA peak
FP6_FP4_PEAK_TFLOPS = 10100.0  # MI355X dense fp6 / fp4 MFMA peak
HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llm")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bwd", action="store_true", help="time only quantize + forward")
    ap.add_argument("--traffic-run", action="store_true",
                    help="for HBM counters: one 1 GiB device copy (calibration), then one mx_attn_bwd call")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "mxfp8_attn_bwd_llm_hbm_traffic.txt")
BWD_SOURCE = os.path.join(ROOT, "mxfp8_block_scaled_flash_amd", "csrc", "attn_bwd.hip")


def source_digest(path):
    """Digest of a source file's code and of the extra flags it is built with: line comments,
    trailing blanks and empty lines removed, so that an edit to the comments does not void counters
    taken on the same code, while a change of its build flags does."""
    import hashlib
    from mxfp8_block_scaled_flash_amd import build as mxbuild
    lines = []
    for line in open(path).read().split("\n"):
        line = line.split("//", 1)[0].rstrip()
        if line.strip():
            lines.append(line)
    lines.append("flags: " + " ".join(mxbuild.FILE_FLAGS.get(os.path.basename(path), [])))
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per mx_attn_bwd call from the committed counter summary, or None when the
    backward's source has changed since the counters were taken."""
    try:
        kv = dict(line[2:].split("=", 1) for line in open(TRAFFIC_FILE) if line.startswith("# ") and "=" in line)
    except OSError:
        return None
    if kv.get("code_sha256_16", "").strip() != source_digest(BWD_SOURCE):
        return None
    return float(kv["bytes_per_call"])


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, sigma):
    """The oracle, as it stands, on a bounded sample of the same workload, on the host's cores.

    Sample: the workload's seeded 4 (batch, head) pairs; per pair the forward of the last 2048
    query rows (the rows with the most visible keys, two chunks of 1024) and the backward of the
    last 4 query blocks (dQ) and the first 4 key blocks (dK, dV).  The work items run on a pool of
    threads (numpy releases the interpreter lock inside its array operations; BLAS is held to one
    thread per item), one per core of this machine's CPU share (at most 16).  FLOPs are counted like
    the GPU's over the visible pairs each item covers: 4 D per pair for the forward, 6 D for a
    query block's backward (S, dP, dQ) and 8 D for a key block's (S, dP, dV, dK)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import synth
    from oracle import attention as at
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    try:
        avail = len(os.sched_getaffinity(0))
    except Exception:
        avail = os.cpu_count() or 1
    nthreads = max(1, min(16, avail))
    S, D = w.S, w.D
    pairs = synth.draw_sample_pairs(w.seed, w.B, w.H, 4)
    heads = {}
    for b, h in pairs:
        q, k, v, do = (synth.head_slice_np(w, t, b, h).double().numpy() for t in ("q", "k", "v", "do"))
        heads[(b, h)] = (q, k, v, do)
    # the backward needs O and LSE of every query: the sample's own forward provides them only for
    # the rows it covers, so the backward items take O = 0 and LSE = log(visible keys) (the uniform
    # softmax's), inputs of the right scale for the oracle's arithmetic
    lse = np.log(np.arange(1, S + 1, dtype=np.float64))
    zero_o = np.zeros((S, D))

    def fwd_item(bh, r0, r1):
        q, k, v, _ = heads[bh]
        at.forward_head(q[:r1], k[:r1], v[:r1], sigma, True, q_rows=np.arange(r0, r1))
        return 4.0 * D * float(np.sum(np.arange(r0, r1) + 1))

    def bwd_item(bh, qb, kb):
        q, k, v, do = heads[bh]
        at.backward_head_blocks(q, k, v, zero_o, do, lse, sigma, True, q_blocks=qb, k_blocks=kb)
        fl = sum(6.0 * D * float(np.sum(np.arange(32 * i, 32 * i + 32) + 1)) for i in qb)
        return fl + sum(8.0 * D * float(np.sum(S - np.arange(32 * j, 32 * j + 32))) for j in kb)

    nb = S // 32
    items = [(fwd_item, (bh, S - 1024 * (i + 1), S - 1024 * i)) for bh in pairs for i in range(2)]
    items += [(bwd_item, (bh, [nb - 1 - i], [])) for bh in pairs for i in range(4)]
    items += [(bwd_item, (bh, [], [i])) for bh in pairs for i in range(4)]
    limit = threadpool_limits(1) if threadpool_limits else None
    try:
        t0 = time.perf_counter()
        with ThreadPoolExecutor(nthreads) as ex:
            flops = sum(ex.map(lambda it: it[0](*it[1]), items))
        dt = time.perf_counter() - t0
    finally:
        if limit is not None:
            limit.unregister()
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": nthreads, "kind": "oracle",
            "sample": f"oracle (numpy, float64) on the B8 H32 S8192 D128 causal workload's 4 sampled (batch, head) "
                      f"pairs {pairs}: forward of the last 2048 query rows and backward of the last 4 query blocks "
                      f"and the first 4 key blocks of each; {len(items)} work items on {nthreads} threads, "
                      f"{dt:.1f} s wall, {flops / 1e12:.3f} TFLOP; CPU: {_cpu_model()}, {avail} cores visible"}


def _bwd_available(mx) -> bool:
    """mx_attn_bwd returns MX_EUNSUPPORTED (2) in builds without the backward."""
    st = mx.lib().mx_attn_bwd(*([None] * 10), 1, None, 1, 32, 1, 128, 0.1, 1, 0, None, None, None, 1, None, 0, None)
    return st != 2


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the workload shards by "
              "(batch, head) with no exchange, so N GPUs would each run this same kernel on B*H/N heads.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import mxfp8_block_scaled_flash_amd as mx
    import synth

    w = synth.workload(args.workload)
    dev = "cuda"
    if args.traffic_run:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    if not args.no_bwd and mx.mx_attn_bwd_workspace_bytes(1, 1, 128) and not _bwd_available(mx):
        print("note: this build's mx_attn_bwd is not available; timing quantize + forward only", file=sys.stderr)
        args.no_bwd = True
    B, S, H, D = w.B, w.S, w.H, w.D
    sigma = 1.0 / math.sqrt(D)
    x = {t: synth.tensor_torch(w, t, dev) for t in ("q", "k", "v", "do")}
    do_bwd = not args.no_bwd
    ROW, COL, SQ = mx.ROW32, mx.COL32, mx.SQ32
    lay = {"q": ROW | SQ, "k": ROW | SQ, "v": COL | ROW, "do": SQ} if do_bwd else {"q": ROW, "k": ROW, "v": COL}
    qz = {t: mx.alloc_quantized(x[t].shape, lay[t], dev) for t in lay}
    o = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=dev)
    if do_bwd:
        dq, dk, dv = (torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev) for _ in range(3))
        ws = torch.empty(mx.mx_attn_bwd_workspace_bytes(B * S, H, D), dtype=torch.uint8, device=dev)

    def g(t, l, i):
        return qz[t][l][i] if l in qz[t] else None

    def quantize_all():
        for t in lay:
            mx.mx_quantize(x[t], B, S, H, D, lay[t], g(t, ROW, 0), g(t, ROW, 1), g(t, COL, 0), g(t, COL, 1),
                           g(t, SQ, 0), g(t, SQ, 1))

    def forward():
        mx.mx_attn_fwd(qz["q"][ROW][0], qz["q"][ROW][1], qz["k"][ROW][0], qz["k"][ROW][1], qz["v"][COL][0],
                       qz["v"][COL][1], B, S, H, D, sigma, True, o, lse)

    def backward():
        mx.mx_attn_bwd(qz["q"][SQ][0], qz["q"][SQ][1], qz["k"][SQ][0], qz["k"][SQ][1], qz["v"][ROW][0],
                       qz["v"][ROW][1], qz["do"][SQ][0], qz["do"][SQ][1], o, x["do"], lse, B, S, H, D, sigma, True,
                       8, dq, dk, dv, ws)

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    def step(rec):
        e = [ev() for _ in range(4)]
        e[0].record(stream)
        quantize_all()
        e[1].record(stream)
        forward()
        e[2].record(stream)
        if do_bwd:
            backward()
        e[3].record(stream)
        if rec is not None:
            rec.append(e)

    if args.traffic_run:
        quantize_all()
        forward()
        if do_bwd:
            backward()
        torch.cuda.synchronize()
        print("traffic run done", flush=True)
        return
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    recs = []
    t_start, t_end = ev(), ev()
    t_start.record(stream)
    for _ in range(args.steps):
        step(recs)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    q_ms = sum(r[0].elapsed_time(r[1]) for r in recs) / len(recs)
    f_ms = sum(r[1].elapsed_time(r[2]) for r in recs) / len(recs)
    b_ms = sum(r[2].elapsed_time(r[3]) for r in recs) / len(recs) if do_bwd else 0.0
    ms_step = total_ms / args.steps

    # fused RMSNorm + quantize (the upstream producer of the Q / K operands; outside the step):
    # Q through ROW32 + SQ32, timed alone on the same stream
    gamma = torch.ones(D, dtype=torch.float32, device="cuda")
    rq = mx.alloc_quantized(x["q"].shape, ROW | SQ, x["q"].device)

    def rmsnorm_q():
        mx.mx_rmsnorm_quantize(x["q"], gamma, 1e-6, B, S, H, D, ROW | SQ, rq[ROW][0], rq[ROW][1], None, None,
                               rq[SQ][0], rq[SQ][1])

    rmsnorm_q()
    r0, r1 = ev(), ev()
    r0.record(stream)
    for _ in range(5):
        rmsnorm_q()
    r1.record(stream)
    torch.cuda.synchronize()
    n_ms = r0.elapsed_time(r1) / 5

    # fused GEMM + quantize (the projection that produces Q; outside the step): tokens x (H D) from a
    # hidden state of width H D, MX operands made by the quantizer, C written as ROW32 + SQ32
    gM, gN, gK = B * S, H * D, H * D
    hid = torch.randn((1, gM, gK // 128, 128), device=dev, dtype=torch.bfloat16)
    wgt = torch.randn((1, gN, gK // 128, 128), device=dev, dtype=torch.bfloat16) * (1.0 / math.sqrt(gK))
    ga, gb = mx.alloc_quantized(hid.shape, ROW, dev), mx.alloc_quantized(wgt.shape, ROW, dev)
    mx.mx_quantize(hid, 1, gM, gK // 128, 128, ROW, ga[ROW][0], ga[ROW][1], None, None, None, None)
    mx.mx_quantize(wgt, 1, gN, gK // 128, 128, ROW, gb[ROW][0], gb[ROW][1], None, None, None, None)
    del hid, wgt
    gc = {l: (torch.empty((gM, gN), dtype=torch.uint8, device=dev),
              torch.empty(((gM, (gN + 31) // 32) if l == ROW else ((gM + 31) // 32, (gN + 31) // 32)),
                          dtype=torch.uint8, device=dev)) for l in (ROW, SQ)}

    def gemm_q():
        mx.mx_gemm_quantize(ga[ROW][0], ga[ROW][1], gb[ROW][0], gb[ROW][1], mx.E4M3, gM, gN, gK, ROW | SQ, gc[ROW][0],
                            gc[ROW][1], None, None, gc[SQ][0], gc[SQ][1], None)

    gemm_q()
    r0, r1 = ev(), ev()
    r0.record(stream)
    for _ in range(5):
        gemm_q()
    r1.record(stream)
    torch.cuda.synchronize()
    g_ms = r0.elapsed_time(r1) / 5
    g_tflops = 2.0 * gM * gN * gK / (g_ms * 1e-3) / 1e12
    # the same GEMM with MXFP6 (E2M3) and MXFP4 (E2M1) operands, produced by the row quantizer
    g_fmt = {}
    hid = torch.randn((gM, gK), device=dev, dtype=torch.bfloat16)
    wgt = torch.randn((gN, gK), device=dev, dtype=torch.bfloat16) * (1.0 / math.sqrt(gK))
    for name, fmt in (("mxfp6_e2m3", mx.E2M3), ("mxfp4_e2m1", mx.E2M1)):
        qa, qb = mx.quantize_rows(hid, fmt), mx.quantize_rows(wgt, fmt)

        def gemm_f(qa=qa, qb=qb, fmt=fmt):
            mx.mx_gemm_quantize(qa[0], qa[1], qb[0], qb[1], fmt, gM, gN, gK, ROW | SQ, gc[ROW][0], gc[ROW][1],
                                None, None, gc[SQ][0], gc[SQ][1], None)

        gemm_f()
        r0, r1 = ev(), ev()
        r0.record(stream)
        for _ in range(5):
            gemm_f()
        r1.record(stream)
        torch.cuda.synchronize()
        ms_ = r0.elapsed_time(r1) / 5
        tf = 2.0 * gM * gN * gK / (ms_ * 1e-3) / 1e12
        g_fmt[name] = {"ms": round(ms_, 4), "tflops": round(tf, 2), "pct_peak": round(100 * tf / FP6_FP4_PEAK_TFLOPS, 2)}
        del qa, qb
    del hid, wgt

    # the forward with Q and K in MXFP6 / MXFP4 (P and V MXFP8) on the same inputs, timed alone
    fwd_fmt = {}
    of = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev)
    for name, fmt in (("mxfp6_e2m3", mx.E2M3), ("mxfp6_e3m2", mx.E3M2), ("mxfp4_e2m1", mx.E2M1)):
        qf, kf = mx.quantize_rows(x["q"].view(-1, D), fmt), mx.quantize_rows(x["k"].view(-1, D), fmt)

        def fwd_f(qf=qf, kf=kf, fmt=fmt):
            mx.mx_attn_fwd_fmt(qf[0], qf[1], kf[0], kf[1], qz["v"][COL][0], qz["v"][COL][1], B, S, H, D, sigma,
                               True, fmt, of, lse)

        fwd_f()
        r0, r1 = ev(), ev()
        r0.record(stream)
        for _ in range(5):
            fwd_f()
        r1.record(stream)
        torch.cuda.synchronize()
        ms_ = r0.elapsed_time(r1) / 5
        fwd_fmt[name] = {"ms": round(ms_, 4), "tflops": round(4.0 * D * B * H * S * (S + 1) / 2 / (ms_ * 1e-3) / 1e12, 2)}
        del qf, kf
    del of

    # the backward with Q and K in MXFP6 / MXFP4 (square blocks; dO, V, P, dS MXFP8) on the same
    # inputs and the step's O and LSE, timed alone
    bwd_fmt = {}
    if do_bwd:
        for name, fmt in (("mxfp6_e2m3", mx.E2M3), ("mxfp4_e2m1", mx.E2M1)):
            qf, kf = mx.quantize_sq_fmt(x["q"], fmt), mx.quantize_sq_fmt(x["k"], fmt)

            def bwd_f(qf=qf, kf=kf, fmt=fmt):
                mx.mx_attn_bwd_fmt(qf[0], qf[1], qf[2], kf[0], kf[1], kf[2], qz["v"][ROW][0], qz["v"][ROW][1],
                                   qz["do"][SQ][0], qz["do"][SQ][1], o, x["do"], lse, B, S, H, D, sigma, True, 8, fmt,
                                   dq, dk, dv, ws)

            bwd_f()
            r0, r1 = ev(), ev()
            r0.record(stream)
            for _ in range(3):
                bwd_f()
            r1.record(stream)
            torch.cuda.synchronize()
            ms_ = r0.elapsed_time(r1) / 3
            bwd_fmt[name] = {"ms": round(ms_, 4),
                             "tflops": round(10.0 * D * B * H * S * (S + 1) / 2 / (ms_ * 1e-3) / 1e12, 2)}
            del qf, kf

    # BF16 attention forward on the same inputs (the baseline of the MX speed-up), timed alone
    o16 = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev)

    def fwd_bf16():
        mx.mx_attn_fwd_bf16(x["q"], x["k"], x["v"], B, S, H, D, sigma, True, o16, lse)

    fwd_bf16()
    r0, r1 = ev(), ev()
    r0.record(stream)
    for _ in range(3):
        fwd_bf16()
    r1.record(stream)
    torch.cuda.synchronize()
    f16_ms = r0.elapsed_time(r1) / 3

    b16_ms = None
    if do_bwd:
        # BF16 attention backward on the same bf16 inputs (O and LSE from the BF16 forward)
        dq16, dk16, dv16 = (torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev) for _ in range(3))
        ws16 = torch.empty(mx.mx_attn_bwd_bf16_workspace_bytes(B * S, H), dtype=torch.uint8, device=dev)
        lse16 = torch.empty((B, H, S), dtype=torch.float32, device=dev)
        mx.mx_attn_fwd_bf16(x["q"], x["k"], x["v"], B, S, H, D, sigma, True, o16, lse16)

        def bwd_bf16():
            mx.mx_attn_bwd_bf16(x["q"], x["k"], x["v"], o16, x["do"], lse16, B, S, H, D, sigma, True, dq16, dk16,
                                dv16, ws16)

        bwd_bf16()
        r0, r1 = ev(), ev()
        r0.record(stream)
        for _ in range(2):
            bwd_bf16()
        r1.record(stream)
        torch.cuda.synchronize()
        b16_ms = r0.elapsed_time(r1) / 2
        del dq16, dk16, dv16, ws16

    pairs = B * H * S * (S + 1) / 2
    f_flop = 4.0 * D * pairs
    b_flop = 10.0 * D * pairs if do_bwd else 0.0
    f_tflops = f_flop / (f_ms * 1e-3) / 1e12
    b_tflops = b_flop / (b_ms * 1e-3) / 1e12 if do_bwd else None
    value = (f_flop + b_flop) / (ms_step * 1e-3) / 1e12
    # quantize: algorithmic bytes = bf16 read + per layout (payload + scales)
    elems = B * S * H * D
    per_layout = {ROW: 1 + 1 / 32, COL: 1 + 1 / 32, SQ: 1 + 1 / 1024}
    q_bytes = sum(elems * (2 + sum(per_layout[l] for l in (ROW, COL, SQ) if lay[t] & l)) for t in lay)

    if do_bwd:
        dom = {"kernel": "mx_attn_bwd (all kernels of the call)", "ms": b_ms, "flop": b_flop}
    else:
        dom = {"kernel": "attn_fwd_kernel", "ms": f_ms, "flop": f_flop}
    achieved = dom["flop"] / (dom["ms"] * 1e-3) / 1e12
    out = {
        "metric": "MXFP8 attn TFLOP/s fwd & bwd, B8 H32 S8192 D128 causal; % of MXFP8 peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8-e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": f"mxfp8 attention fwd+bwd B{B} H{H} S{S} D{D} causal bf16 N(0,1)",
                   "B": B, "H": H, "S": S, "D": D, "causal": True},
        "fwd_tflops": round(f_tflops, 2),
        "fwd_pct_peak": round(100 * f_tflops / MXFP8_PEAK_TFLOPS, 2),
        "bwd_tflops": round(b_tflops, 2) if b_tflops else None,
        "bwd_pct_peak": round(100 * b_tflops / MXFP8_PEAK_TFLOPS, 2) if b_tflops else None,
        "quantize_ms": round(q_ms, 4),
        "quantize_gbs": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
        "rmsnorm_quantize_ms": round(n_ms, 4),
        "rmsnorm_quantize_gbs": round(B * S * H * D * (2 + per_layout[ROW] + per_layout[SQ]) / (n_ms * 1e-3) / 1e9, 1),
        "gemm_quantize": {"M": gM, "N": gN, "K": gK, "layouts": "row32+sq32", "ms": round(g_ms, 4),
                          "tflops": round(g_tflops, 2), "pct_peak": round(100 * g_tflops / MXFP8_PEAK_TFLOPS, 2),
                          **g_fmt},
        "fwd_qk_formats": fwd_fmt,
        "bwd_qk_formats": bwd_fmt,
        "bf16_fwd": {"ms": round(f16_ms, 4), "tflops": round(f_flop / (f16_ms * 1e-3) / 1e12, 2),
                     "pct_bf16_peak": round(100 * f_flop / (f16_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
                     "mx_speedup": round(f16_ms / f_ms, 3)},
        "bf16_bwd": ({"ms": round(b16_ms, 4), "tflops": round(b_flop / (b16_ms * 1e-3) / 1e12, 2),
                      "pct_bf16_peak": round(100 * b_flop / (b16_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 2),
                      "mx_speedup": round(b16_ms / b_ms, 3)} if b16_ms else None),
        "fwd_ms": round(f_ms, 4),
        "bwd_ms": round(b_ms, 4) if do_bwd else None,
        "roofline": {"bound": "mfma", "kernel": dom["kernel"], "achieved": round(achieved, 2),
                     "peak": MXFP8_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / MXFP8_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic() if do_bwd else None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, sigma)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
