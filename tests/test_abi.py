"""The C-ABI library: it loads, exports every entry point the header
declares, and rejects invalid arguments on the host before launching
anything (these calls need no GPU)."""
import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_flash_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfa.h")
EINVAL, EWORKSPACE = 1, 4


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mx_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared() == mx.exported_symbols()


def test_library_exports_every_declared_symbol():
    L = mx.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.mx_abi_version() == 1
    for s in range(5):
        assert L.mx_status_str(s).decode().startswith("MX_")


def _quant(**kw):
    args = dict(x=16, dt=mx.BF16, B=1, S=32, H=1, D=128, lay=mx.ROW32, rd=16, rs=16, cd=None, cs=None, sd=None,
                ss=None)
    args.update(kw)
    return mx.lib().mx_quantize(args["x"], args["dt"], args["B"], args["S"], args["H"], args["D"], args["lay"],
                                args["rd"], args["rs"], args["cd"], args["cs"], args["sd"], args["ss"], None)


@pytest.mark.parametrize("bad", [dict(D=96), dict(D=0), dict(H=0), dict(B=-1), dict(S=-3), dict(lay=0),
                                 dict(lay=8), dict(dt=mx.F16), dict(x=None), dict(x=24), dict(rd=None),
                                 dict(rs=8), dict(lay=mx.COL32), dict(lay=mx.SQ32 | mx.ROW32)])
def test_quantize_rejects_invalid_arguments(bad):
    assert _quant(**bad) == EINVAL


def test_empty_quantize_is_a_no_op():
    assert _quant(B=0) == 0 and _quant(S=0) == 0


def _fwd(**kw):
    a = dict(q=16, qs=16, k=16, ks=16, v=16, vs=16, B=1, S=64, H=1, D=128, sc=0.1, causal=1, o=16, odt=mx.BF16,
             lse=None)
    a.update(kw)
    return mx.lib().mx_attn_fwd(a["q"], a["qs"], a["k"], a["ks"], a["v"], a["vs"], a["B"], a["S"], a["H"], a["D"],
                                a["sc"], a["causal"], a["o"], a["odt"], a["lse"], None)


@pytest.mark.parametrize("bad", [dict(B=2, S=1 << 30), dict(H=(1 << 16) + 1, S=32)])
def test_forward_rejects_sizes_past_the_index_range(bad):
    # 2^31 tokens, or more heads than a tile's 32-bit byte span allows: rejected on the host
    assert _fwd(**bad) == EINVAL


@pytest.mark.parametrize("bad", [dict(D=32), dict(H=0), dict(S=-1), dict(sc=0.0), dict(sc=-1.0),
                                 dict(sc=float("nan")), dict(sc=float("inf")), dict(odt=mx.F16), dict(o=None),
                                 dict(q=None), dict(vs=4), dict(lse=4)])
def test_forward_rejects_invalid_arguments(bad):
    assert _fwd(**bad) == EINVAL


@pytest.mark.parametrize("fmt", [1, 5, -1])
def test_forward_fmt_rejects_unknown_formats(fmt):
    # qk_format is checked before anything touches the device
    assert mx.lib().mx_attn_fwd_fmt(*([16] * 6), 1, 64, 1, 128, 0.1, 1, fmt, 16, mx.BF16, None, None) == EINVAL


@pytest.mark.parametrize("fmt", [1, 5])
def test_forward_fmt_varlen_rejects_unknown_formats(fmt):
    assert mx.lib().mx_attn_fwd_fmt_varlen(*([16] * 6), 16, 16, 1, 10, 10, 1, 128, 0.1, 1, fmt, 16, mx.BF16, None,
                                           None) == EINVAL


@pytest.mark.parametrize("bad", [dict(D=32), dict(H=0), dict(S=-1), dict(sc=0.0), dict(o=None), dict(q=None)])
def test_forward_fmt_rejects_invalid_arguments(bad):
    a = dict(q=16, B=1, S=64, H=1, D=128, sc=0.1, o=16)
    a.update(bad)
    assert mx.lib().mx_attn_fwd_fmt(a["q"], 16, 16, 16, 16, 16, a["B"], a["S"], a["H"], a["D"], a["sc"], 1, mx.E2M1,
                                    a["o"], mx.BF16, None, None) == EINVAL


def test_varlen_rejects_invalid_arguments():
    L = mx.lib()
    # total_scale_rows not a multiple of 128, and smaller than the token count
    assert L.mx_quantize_varlen(16, mx.BF16, 16, 16, 1, 10, 100, 1, 128, 1, 16, 16, None, None, None, None,
                                None) == EINVAL
    assert L.mx_quantize_varlen(16, mx.BF16, 16, 16, 1, 300, 256, 1, 128, 1, 16, 16, None, None, None, None,
                                None) == EINVAL
    assert L.mx_quantize_varlen(16, mx.BF16, None, 16, 1, 10, 128, 1, 128, 1, 16, 16, None, None, None, None,
                                None) == EINVAL
    assert L.mx_varlen_scale_offsets(None, 1, 16, None) == EINVAL
    assert L.mx_varlen_scale_offsets(16, 0, 16, None) == EINVAL
    assert L.mx_attn_fwd_varlen(*([16] * 6), 16, 16, 0, 10, 10, 1, 128, ctypes.c_float(0.1), 1, 16, mx.BF16,
                                None, None) == EINVAL


@pytest.mark.parametrize("gamma,eps", [(None, 1e-6), (16, -1.0), (16, float("nan")), (16, float("inf")), (18, 1e-6)])
def test_rmsnorm_quantize_rejects_invalid_norm_arguments(gamma, eps):
    L = mx.lib()
    # null or misaligned gain, negative or non-finite epsilon: rejected before any device work
    assert L.mx_rmsnorm_quantize(16, mx.BF16, gamma, eps, 1, 32, 1, 128, mx.ROW32, 16, 16, None, None, None, None,
                                 None) == EINVAL
    assert L.mx_rmsnorm_quantize_varlen(16, mx.BF16, gamma, eps, 16, 16, 1, 10, 128, 1, 128, mx.ROW32, 16, 16,
                                        None, None, None, None, None) == EINVAL


def test_rmsnorm_quantize_rejects_invalid_shapes():
    L = mx.lib()
    assert L.mx_rmsnorm_quantize(16, mx.BF16, 16, 1e-6, 1, 32, 1, 96, mx.ROW32, 16, 16, None, None, None, None,
                                 None) == EINVAL
    assert L.mx_rmsnorm_quantize(16, mx.F16, 16, 1e-6, 1, 32, 1, 128, mx.ROW32, 16, 16, None, None, None, None,
                                 None) == EINVAL
    assert L.mx_rmsnorm_quantize(16, mx.BF16, 16, 1e-6, 1, 32, 1, 128, 0, 16, 16, None, None, None, None,
                                 None) == EINVAL


def _gemm(**kw):
    a = dict(a=16, as_=16, b=16, bs=16, fmt=mx.E4M3, M=64, N=64, K=64, lay=mx.ROW32, rd=16, rs=16, cd=None, cs=None,
             sd=None, ss=None, c32=None)
    a.update(kw)
    return mx.lib().mx_gemm_quantize(a["a"], a["as_"], a["b"], a["bs"], a["fmt"], a["M"], a["N"], a["K"], a["lay"],
                                     a["rd"],
                                     a["rs"], a["cd"], a["cs"], a["sd"], a["ss"], a["c32"], None)


@pytest.mark.parametrize("bad", [dict(K=32), dict(K=0), dict(K=96), dict(N=40), dict(M=-1), dict(N=-16),
                                 dict(lay=8), dict(lay=0), dict(a=None), dict(bs=24), dict(rd=None),
                                 dict(lay=mx.COL32), dict(c32=20), dict(K=(1 << 20) + 64), dict(fmt=1), dict(fmt=5)])
def test_gemm_quantize_rejects_invalid_arguments(bad):
    assert _gemm(**bad) == EINVAL


def test_empty_gemm_quantize_is_a_no_op():
    assert _gemm(M=0) == 0 and _gemm(N=0) == 0 and _gemm(M=0, lay=0, rd=None, rs=None, c32=16) == 0


def _fwd16(**kw):
    a = dict(q=16, k=16, v=16, B=1, S=64, H=1, D=128, sc=0.1, causal=1, o=16, odt=mx.BF16, lse=None)
    a.update(kw)
    return mx.lib().mx_attn_fwd_bf16(a["q"], a["k"], a["v"], a["B"], a["S"], a["H"], a["D"], a["sc"], a["causal"],
                                     a["o"], a["odt"], a["lse"], None)


@pytest.mark.parametrize("bad", [dict(D=96), dict(H=0), dict(B=-1), dict(sc=0.0), dict(sc=float("inf")),
                                 dict(odt=mx.F16), dict(q=None), dict(v=24), dict(o=8), dict(lse=20)])
def test_bf16_forward_rejects_invalid_arguments(bad):
    assert _fwd16(**bad) == EINVAL


def test_bf16_forward_empty_and_varlen_validation():
    assert _fwd16(B=0) == 0 and _fwd16(S=0) == 0
    L = mx.lib()
    assert L.mx_attn_fwd_bf16_varlen(16, 16, 16, None, 1, 10, 10, 1, 128, 0.1, 1, 16, mx.BF16, None, None) == EINVAL
    assert L.mx_attn_fwd_bf16_varlen(16, 16, 16, 16, 0, 10, 10, 1, 128, 0.1, 1, 16, mx.BF16, None, None) == EINVAL
    assert L.mx_attn_fwd_bf16_varlen(16, 16, 16, 16, 1, 0, 10, 1, 128, 0.1, 1, 16, mx.BF16, None, None) == 0


def test_bf16_backward_validation():
    L = mx.lib()
    n = L.mx_attn_bwd_bf16_workspace_bytes(64, 2)
    assert n == 512 and L.mx_attn_bwd_bf16_workspace_bytes(-1, 2) == 0
    args = [16] * 6 + [1, 64, 1, 128, 0.1, 1] + [16] * 3 + [mx.BF16, 16, n, None]

    def call(**kw):
        a = list(args)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return L.mx_attn_bwd_bf16(*a)
    assert call(a9=80) == EINVAL and call(a10=0.0) == EINVAL and call(a15=mx.F16) == EINVAL
    assert call(a0=None) == EINVAL and call(a5=24) == EINVAL
    assert call(a16=None) == 4 and call(a17=L.mx_attn_bwd_bf16_workspace_bytes(64, 1) - 1) == 4
    assert call(a6=0) == 0


def test_quantize_rows_validation():
    L = mx.lib()
    ok = dict(x=16, dt=mx.BF16, rows=4, K=64, fmt=mx.E2M1, d=16, s=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.mx_quantize_rows(a["x"], a["dt"], a["rows"], a["K"], a["fmt"], a["d"], a["s"], None)
    for bad in (dict(K=48), dict(K=0), dict(rows=-1), dict(fmt=1), dict(fmt=7), dict(dt=mx.F16), dict(x=None),
                dict(d=24), dict(s=None)):
        assert call(**bad) == EINVAL, bad
    assert call(rows=0) == 0


def test_workspace_size():
    n = mx.lib().mx_attn_bwd_workspace_bytes(1000, 3, 128)
    assert n >= 1000 * 3 * 128 * 2 + 1000 * 3 * 4 and n % 256 == 0
    assert mx.lib().mx_attn_bwd_workspace_bytes(-1, 3, 128) == 0


def test_library_has_no_unresolved_kernel_stubs():
    import subprocess
    out = subprocess.run(["nm", "-D", mx._LIB_PATH], capture_output=True, text=True).stdout
    missing = [l for l in out.splitlines() if " U " in l and "__device_stub__" in l]
    assert not missing, missing


def test_workspace_layout_has_the_range_flag_slot():
    # 256-byte flag slot + fp16 accumulator + D_i, each 256-byte aligned
    assert mx.lib().mx_attn_bwd_workspace_bytes(64, 1, 128) == 256 + 64 * 128 * 2 + 256
    assert mx.lib().mx_attn_bwd_workspace_bytes(0, 1, 128) == 256


def test_mx_backward_rejects_invalid_arguments():
    """mx_attn_bwd checks shapes, dtypes, the softmax and dQ scales, pointers and the workspace on
    the host, before anything touches a device."""
    L = mx.lib()
    n = L.mx_attn_bwd_workspace_bytes(64, 1, 128)
    args = [16] * 8 + [16, 16, mx.BF16, 16, 1, 64, 1, 128, 0.1, 1, 8, 16, 16, 16, mx.BF16, 16, n, None]

    def call(**kw):
        a = list(args)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return L.mx_attn_bwd(*a)
    for bad in (dict(a15=96), dict(a14=0), dict(a12=-1), dict(a13=-5), dict(a16=0.0), dict(a16=float("nan")),
                dict(a18=16), dict(a18=-16), dict(a10=mx.F16), dict(a22=mx.F16), dict(a0=None), dict(a7=None),
                dict(a8=None), dict(a11=None), dict(a19=None), dict(a3=24), dict(a9=40), dict(a14=(1 << 16) + 1),
                dict(a12=2, a13=1 << 30)):
        assert call(**bad) == EINVAL, bad
    assert call(a23=None) == EWORKSPACE and call(a23=24) == EWORKSPACE and call(a24=n - 1) == EWORKSPACE
    assert call(a12=0) == 0 and call(a13=0) == 0


def test_mx_backward_varlen_rejects_invalid_arguments():
    L = mx.lib()
    n = L.mx_attn_bwd_workspace_bytes(64, 1, 128)
    args = [16] * 8 + [16, 16, mx.BF16, 16, 16, 16, 2, 64, 40, 1, 128, 0.1, 1, 8, 16, 16, 16, mx.BF16, 16, n, None]

    def call(**kw):
        a = list(args)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return L.mx_attn_bwd_varlen(*a)
    for bad in (dict(a12=None), dict(a13=None), dict(a14=0), dict(a15=-1), dict(a16=-1), dict(a18=80),
                dict(a19=-1.0), dict(a21=20), dict(a10=mx.F16), dict(a0=None), dict(a22=None)):
        assert call(**bad) == EINVAL, bad
    assert call(a26=None) == EWORKSPACE and call(a27=n - 1) == EWORKSPACE
    assert call(a15=0) == 0 and call(a16=0) == 0


def test_overflow_query_rejects_bad_pointers():
    L = mx.lib()
    flag = ctypes.c_int(0)
    assert L.mx_attn_bwd_overflow(16, None, None) == EINVAL
    assert L.mx_attn_bwd_overflow(24, ctypes.byref(flag), None) == EINVAL
    assert L.mx_attn_bwd_overflow(None, None, None) == EINVAL


def test_noalloc_backward_rejects_invalid_and_oversized_calls_before_the_device():
    """mx_attn_bwd_noalloc validates like mx_attn_bwd (no workspace arguments) and rejects calls
    whose scratch would exceed MX_NOALLOC_MAX_BYTES (128 MiB) with MX_EWORKSPACE, all on the host."""
    L = mx.lib()
    args = [16] * 8 + [16, 16, mx.BF16, 16, 1, 64, 1, 128, 0.1, 1, 8, 16, 16, 16, mx.BF16, None]

    def call(**kw):
        a = list(args)
        for i, val in kw.items():
            a[int(i[1:])] = val
        return L.mx_attn_bwd_noalloc(*a)
    for bad in (dict(a15=96), dict(a14=0), dict(a12=-1), dict(a16=0.0), dict(a18=16), dict(a10=mx.F16),
                dict(a0=None), dict(a11=None), dict(a3=24)):
        assert call(**bad) == EINVAL, bad
    assert call(a12=0) == 0
    # the long-context workload (B4 S4096 H16 D128) and B2 S8192 H16 fit; B4 S8192 H16 does not
    assert L.mx_attn_bwd_workspace_bytes(4 * 4096, 16, 128) <= 128 << 20
    assert L.mx_attn_bwd_workspace_bytes(2 * 8192, 16, 128) <= 128 << 20
    assert call(a12=4, a13=8192, a14=16) == EWORKSPACE
    assert call(a12=8, a13=8192, a14=32) == EWORKSPACE


def test_quantize_rows_varlen_validation():
    L = mx.lib()
    ok = dict(x=16, dt=mx.BF16, cu=16, csr=16, nseq=2, T=100, Tp=256, H=2, K=64, fmt=mx.E2M1, d=16, s=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.mx_quantize_rows_varlen(a["x"], a["dt"], a["cu"], a["csr"], a["nseq"], a["T"], a["Tp"], a["H"],
                                         a["K"], a["fmt"], a["d"], a["s"], None)
    for bad in (dict(cu=None), dict(csr=None), dict(nseq=0), dict(T=-1), dict(Tp=100), dict(Tp=64), dict(K=48),
                dict(fmt=1), dict(dt=mx.F16), dict(H=0), dict(x=None), dict(d=24), dict(s=None)):
        assert call(**bad) == EINVAL, bad
    assert call(T=0) == 0


def test_quantize_sq_fmt_validation():
    L = mx.lib()
    ok = dict(x=16, dt=mx.BF16, B=2, S=40, H=2, D=128, fmt=mx.E2M3, r=16, c=16, s=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.mx_quantize_sq_fmt(a["x"], a["dt"], a["B"], a["S"], a["H"], a["D"], a["fmt"], a["r"], a["c"],
                                    a["s"], None)
    for bad in (dict(D=96), dict(D=32), dict(B=-1), dict(S=-1), dict(H=0), dict(fmt=mx.E4M3), dict(fmt=1),
                dict(dt=mx.F16), dict(x=None), dict(r=None), dict(c=24), dict(s=None)):
        assert call(**bad) == EINVAL, bad
    assert call(B=0) == 0 and call(S=0) == 0


def test_quantize_sq_fmt_varlen_validation():
    L = mx.lib()
    ok = dict(x=16, dt=mx.BF16, cu=16, csr=16, nseq=2, T=100, Tp=256, H=2, D=64, fmt=mx.E2M1, r=16, c=16, s=16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.mx_quantize_sq_fmt_varlen(a["x"], a["dt"], a["cu"], a["csr"], a["nseq"], a["T"], a["Tp"], a["H"],
                                           a["D"], a["fmt"], a["r"], a["c"], a["s"], None)
    for bad in (dict(cu=None), dict(csr=None), dict(nseq=0), dict(T=-1), dict(Tp=100), dict(Tp=64), dict(D=48),
                dict(fmt=mx.E4M3), dict(dt=mx.F16), dict(H=0), dict(x=None), dict(r=24), dict(c=None), dict(s=None)):
        assert call(**bad) == EINVAL, bad
    assert call(T=0) == 0


def test_attn_bwd_fmt_validation():
    """The small-format backward rejects what it cannot take before touching the device: a format
    outside E4M3 / E2M3 / E3M2 / E2M1, D != 128 with a small format, null column-packed payloads."""
    L = mx.lib()
    ws = 1 << 20

    def call(fmt=mx.E2M1, D=128, qc=16, kc=16, B=1, S=64):
        return L.mx_attn_bwd_fmt(16, qc, 16, 16, kc, 16, 16, 16, 16, 16, 16, 16, mx.BF16, 16, B, S, 2, D, 0.125, 1, 8,
                                 fmt, 16, 16, 16, mx.BF16, 16, ws, None)
    for bad in (dict(fmt=1), dict(fmt=5), dict(D=64), dict(qc=None), dict(kc=None), dict(qc=24), dict(B=-1)):
        assert call(**bad) == EINVAL, bad
    assert call(B=0) == 0 and call(S=0) == 0

    def callv(fmt=mx.E2M3, D=128, nseq=2, cu=16):
        return L.mx_attn_bwd_fmt_varlen(16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, 16, mx.BF16, 16, cu, 16, nseq,
                                        100, 64, 2, D, 0.125, 1, 8, fmt, 16, 16, 16, mx.BF16, 16, ws, None)
    for bad in (dict(fmt=7), dict(D=64), dict(nseq=0), dict(cu=None)):
        assert callv(**bad) == EINVAL, bad
