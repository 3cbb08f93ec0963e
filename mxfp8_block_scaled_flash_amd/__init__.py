"""Python binding of libmxfa (MXFP8 block-scaled attention for MI355X).

Argument marshalling only: each ``mx_*`` function below has the name and the
argument order of the C entry point in ``include/mxfa.h``, takes torch
tensors where the C call takes device pointers, passes the current HIP stream,
and raises :class:`MXError` on a non-zero status.  Every step of the
computation runs in the HIP kernels of ``libmxfa.so``; there is no fallback.
The ``alloc_*`` helpers only allocate output tensors of the documented shapes
(PyTorch supplies device memory and streams).
"""
from __future__ import annotations

import ctypes
import os

import torch

ROW32, COL32, SQ32 = 1, 2, 4
F32, BF16, F16 = 0, 1, 2
LAYOUT_NAMES = {ROW32: "row32", COL32: "col32", SQ32: "sq32"}
# element formats (the block-scaled matrix instruction's format codes) and their widths in bits
E4M3, E2M3, E3M2, E2M1 = 0, 2, 3, 4
ELEM_BITS = {E4M3: 8, E2M3: 6, E3M2: 6, E2M1: 4}

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfa.so")
_lib = None

_c_int, _c_size, _c_float, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p

_SIGS = {
    "mx_abi_version": ([], _c_int),
    "mx_status_str": ([_c_int], ctypes.c_char_p),
    "mx_quantize": ([_vp, _c_int, _c_int, _c_int, _c_int, _c_int, ctypes.c_uint] + [_vp] * 6 + [_vp], _c_int),
    "mx_varlen_scale_offsets": ([_vp, _c_int, _vp, _vp], _c_int),
    "mx_quantize_varlen": ([_vp, _c_int, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, ctypes.c_uint]
                           + [_vp] * 6 + [_vp], _c_int),
    "mx_rmsnorm_quantize": ([_vp, _c_int, _vp, _c_float, _c_int, _c_int, _c_int, _c_int, ctypes.c_uint]
                            + [_vp] * 6 + [_vp], _c_int),
    "mx_rmsnorm_quantize_varlen": ([_vp, _c_int, _vp, _c_float, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    ctypes.c_uint] + [_vp] * 6 + [_vp], _c_int),
    "mx_quantize_rows": ([_vp, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp], _c_int),
    "mx_quantize_rows_varlen": ([_vp, _c_int, _vp, _vp] + [_c_int] * 6 + [_vp, _vp, _vp], _c_int),
    "mx_quantize_sq_fmt": ([_vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp], _c_int),
    "mx_quantize_sq_fmt_varlen": ([_vp, _c_int, _vp, _vp] + [_c_int] * 6 + [_vp, _vp, _vp, _vp], _c_int),
    "mx_gemm_quantize": ([_vp] * 4 + [_c_int] * 4 + [ctypes.c_uint] + [_vp] * 7 + [_vp], _c_int),
    "mx_attn_fwd": ([_vp] * 6 + [_c_int] * 4 + [_c_float, _c_int, _vp, _c_int, _vp, _vp], _c_int),
    "mx_attn_fwd_varlen": ([_vp] * 6 + [_vp, _vp] + [_c_int] * 5 + [_c_float, _c_int, _vp, _c_int, _vp, _vp],
                           _c_int),
    "mx_attn_fwd_fmt": ([_vp] * 6 + [_c_int] * 4 + [_c_float, _c_int, _c_int, _vp, _c_int, _vp, _vp], _c_int),
    "mx_attn_fwd_fmt_varlen": ([_vp] * 6 + [_vp, _vp] + [_c_int] * 5 + [_c_float, _c_int, _c_int, _vp, _c_int, _vp,
                                                                      _vp], _c_int),
    "mx_attn_fwd_bf16": ([_vp] * 3 + [_c_int] * 4 + [_c_float, _c_int, _vp, _c_int, _vp, _vp], _c_int),
    "mx_attn_fwd_bf16_varlen": ([_vp] * 4 + [_c_int] * 5 + [_c_float, _c_int, _vp, _c_int, _vp, _vp], _c_int),
    "mx_attn_bwd_workspace_bytes": ([_c_int, _c_int, _c_int], _c_size),
    "mx_attn_bwd_overflow": ([_vp, _vp, _vp], _c_int),
    "mx_attn_bwd_bf16_workspace_bytes": ([_c_int, _c_int], _c_size),
    "mx_attn_bwd_bf16": ([_vp] * 6 + [_c_int] * 4 + [_c_float, _c_int] + [_vp] * 3 + [_c_int, _vp, _c_size, _vp],
                         _c_int),
    "mx_attn_bwd_bf16_varlen": ([_vp] * 6 + [_vp] + [_c_int] * 5 + [_c_float, _c_int] + [_vp] * 3
                                + [_c_int, _vp, _c_size, _vp], _c_int),
    "mx_attn_bwd": ([_vp] * 8 + [_vp, _vp, _c_int, _vp] + [_c_int] * 4 + [_c_float, _c_int, _c_int]
                    + [_vp] * 3 + [_c_int, _vp, _c_size, _vp], _c_int),
    "mx_attn_bwd_fmt": ([_vp] * 10 + [_vp, _vp, _c_int, _vp] + [_c_int] * 4 + [_c_float, _c_int, _c_int, _c_int]
                        + [_vp] * 3 + [_c_int, _vp, _c_size, _vp], _c_int),
    "mx_attn_bwd_fmt_varlen": ([_vp] * 10 + [_vp, _vp, _c_int, _vp] + [_vp, _vp] + [_c_int] * 5
                               + [_c_float, _c_int, _c_int, _c_int] + [_vp] * 3 + [_c_int, _vp, _c_size, _vp], _c_int),
    "mx_attn_bwd_noalloc": ([_vp] * 8 + [_vp, _vp, _c_int, _vp] + [_c_int] * 4 + [_c_float, _c_int, _c_int]
                            + [_vp] * 3 + [_c_int, _vp], _c_int),
    "mx_attn_bwd_varlen": ([_vp] * 8 + [_vp, _vp, _c_int, _vp] + [_vp, _vp] + [_c_int] * 5
                           + [_c_float, _c_int, _c_int] + [_vp] * 3 + [_c_int, _vp, _c_size, _vp], _c_int),
}


class MXError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """Load libmxfa.so (built by ``python -m mxfp8_block_scaled_flash_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m mxfp8_block_scaled_flash_amd.build` (there is no fallback)")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def exported_symbols():
    return sorted(_SIGS)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    if stream is not None:
        return stream
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, what: str):
    if status != 0:
        msg = lib().mx_status_str(status).decode()
        raise MXError(f"{what}: {msg}")


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return F32
    if dt == torch.bfloat16:
        return BF16
    if dt == torch.float16:
        return F16
    raise MXError(f"unsupported dtype {dt}")


# --------------------------------------------------------------- raw entry points
def mx_abi_version() -> int:
    return lib().mx_abi_version()


def mx_quantize(x, B, S, H, D, layouts, row32_data, row32_scale, col32_data, col32_scale, sq32_data, sq32_scale,
                stream=None):
    _check(lib().mx_quantize(_ptr(x), _dtype_code(x.dtype), B, S, H, D, layouts, _ptr(row32_data),
                             _ptr(row32_scale), _ptr(col32_data), _ptr(col32_scale), _ptr(sq32_data),
                             _ptr(sq32_scale), _stream(stream)), "mx_quantize")


def mx_varlen_scale_offsets(cu_seqlens, nseq, cu_scale_rows, stream=None):
    _check(lib().mx_varlen_scale_offsets(_ptr(cu_seqlens), nseq, _ptr(cu_scale_rows), _stream(stream)),
           "mx_varlen_scale_offsets")


def mx_quantize_varlen(x, cu_seqlens, cu_scale_rows, nseq, total_tokens, total_scale_rows, H, D, layouts,
                       row32_data, row32_scale, col32_data, col32_scale, sq32_data, sq32_scale, stream=None):
    _check(lib().mx_quantize_varlen(_ptr(x), _dtype_code(x.dtype), _ptr(cu_seqlens), _ptr(cu_scale_rows), nseq,
                                    total_tokens, total_scale_rows, H, D, layouts, _ptr(row32_data),
                                    _ptr(row32_scale), _ptr(col32_data), _ptr(col32_scale), _ptr(sq32_data),
                                    _ptr(sq32_scale), _stream(stream)), "mx_quantize_varlen")


def mx_rmsnorm_quantize(x, gamma, eps, B, S, H, D, layouts, row32_data, row32_scale, col32_data, col32_scale,
                        sq32_data, sq32_scale, stream=None):
    _check(lib().mx_rmsnorm_quantize(_ptr(x), _dtype_code(x.dtype), _ptr(gamma), float(eps), B, S, H, D, layouts,
                                     _ptr(row32_data), _ptr(row32_scale), _ptr(col32_data), _ptr(col32_scale),
                                     _ptr(sq32_data), _ptr(sq32_scale), _stream(stream)), "mx_rmsnorm_quantize")


def mx_rmsnorm_quantize_varlen(x, gamma, eps, cu_seqlens, cu_scale_rows, nseq, total_tokens, total_scale_rows, H,
                               D, layouts, row32_data, row32_scale, col32_data, col32_scale, sq32_data, sq32_scale,
                               stream=None):
    _check(lib().mx_rmsnorm_quantize_varlen(_ptr(x), _dtype_code(x.dtype), _ptr(gamma), float(eps),
                                            _ptr(cu_seqlens), _ptr(cu_scale_rows), nseq, total_tokens,
                                            total_scale_rows, H, D, layouts, _ptr(row32_data), _ptr(row32_scale),
                                            _ptr(col32_data), _ptr(col32_scale), _ptr(sq32_data), _ptr(sq32_scale),
                                            _stream(stream)), "mx_rmsnorm_quantize_varlen")


def mx_quantize_rows(x, rows, K, fmt, data, scale, stream=None):
    _check(lib().mx_quantize_rows(_ptr(x), _dtype_code(x.dtype), rows, K, fmt, _ptr(data), _ptr(scale),
                                  _stream(stream)), "mx_quantize_rows")


def mx_quantize_rows_varlen(x, cu_seqlens, cu_scale_rows, nseq, total_tokens, total_scale_rows, H, K, fmt, data,
                            scale, stream=None):
    _check(lib().mx_quantize_rows_varlen(_ptr(x), _dtype_code(x.dtype), _ptr(cu_seqlens), _ptr(cu_scale_rows), nseq,
                                         total_tokens, total_scale_rows, H, K, fmt, _ptr(data), _ptr(scale),
                                         _stream(stream)), "mx_quantize_rows_varlen")


def mx_gemm_quantize(a_data, a_scale, b_data, b_scale, fmt, M, N, K, layouts, c_row32_data, c_row32_scale,
                     c_col32_data, c_col32_scale, c_sq32_data, c_sq32_scale, c_f32, stream=None):
    _check(lib().mx_gemm_quantize(_ptr(a_data), _ptr(a_scale), _ptr(b_data), _ptr(b_scale), fmt, M, N, K, layouts,
                                  _ptr(c_row32_data), _ptr(c_row32_scale), _ptr(c_col32_data), _ptr(c_col32_scale),
                                  _ptr(c_sq32_data), _ptr(c_sq32_scale), _ptr(c_f32), _stream(stream)),
           "mx_gemm_quantize")


def mx_attn_fwd(q_data, q_scale, k_data, k_scale, v_data, v_scale, B, S, H, D, softmax_scale, causal, o, lse,
                stream=None):
    _check(lib().mx_attn_fwd(_ptr(q_data), _ptr(q_scale), _ptr(k_data), _ptr(k_scale), _ptr(v_data),
                             _ptr(v_scale), B, S, H, D, float(softmax_scale), int(bool(causal)), _ptr(o),
                             _dtype_code(o.dtype), _ptr(lse), _stream(stream)), "mx_attn_fwd")


def mx_attn_fwd_varlen(q_data, q_scale, k_data, k_scale, v_data, v_scale, cu_seqlens, cu_scale_rows, nseq,
                       total_tokens, max_seqlen, H, D, softmax_scale, causal, o, lse, stream=None):
    _check(lib().mx_attn_fwd_varlen(_ptr(q_data), _ptr(q_scale), _ptr(k_data), _ptr(k_scale), _ptr(v_data),
                                    _ptr(v_scale), _ptr(cu_seqlens), _ptr(cu_scale_rows), nseq, total_tokens,
                                    max_seqlen, H, D, float(softmax_scale), int(bool(causal)), _ptr(o),
                                    _dtype_code(o.dtype), _ptr(lse), _stream(stream)), "mx_attn_fwd_varlen")


def mx_attn_fwd_fmt(q_data, q_scale, k_data, k_scale, v_data, v_scale, B, S, H, D, softmax_scale, causal,
                    qk_format, o, lse, stream=None):
    _check(lib().mx_attn_fwd_fmt(_ptr(q_data), _ptr(q_scale), _ptr(k_data), _ptr(k_scale), _ptr(v_data),
                                 _ptr(v_scale), B, S, H, D, float(softmax_scale), int(bool(causal)), int(qk_format),
                                 _ptr(o), _dtype_code(o.dtype), _ptr(lse), _stream(stream)), "mx_attn_fwd_fmt")


def mx_attn_fwd_fmt_varlen(q_data, q_scale, k_data, k_scale, v_data, v_scale, cu_seqlens, cu_scale_rows, nseq,
                           total_tokens, max_seqlen, H, D, softmax_scale, causal, qk_format, o, lse, stream=None):
    _check(lib().mx_attn_fwd_fmt_varlen(_ptr(q_data), _ptr(q_scale), _ptr(k_data), _ptr(k_scale), _ptr(v_data),
                                        _ptr(v_scale), _ptr(cu_seqlens), _ptr(cu_scale_rows), nseq, total_tokens,
                                        max_seqlen, H, D, float(softmax_scale), int(bool(causal)), int(qk_format),
                                        _ptr(o), _dtype_code(o.dtype), _ptr(lse), _stream(stream)),
           "mx_attn_fwd_fmt_varlen")


def mx_attn_fwd_bf16(q, k, v, B, S, H, D, softmax_scale, causal, o, lse, stream=None):
    _check(lib().mx_attn_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), B, S, H, D, float(softmax_scale), int(bool(causal)),
                                  _ptr(o), _dtype_code(o.dtype), _ptr(lse), _stream(stream)), "mx_attn_fwd_bf16")


def mx_attn_fwd_bf16_varlen(q, k, v, cu_seqlens, nseq, total_tokens, max_seqlen, H, D, softmax_scale, causal, o,
                            lse, stream=None):
    _check(lib().mx_attn_fwd_bf16_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), nseq, total_tokens,
                                         max_seqlen, H, D, float(softmax_scale), int(bool(causal)), _ptr(o),
                                         _dtype_code(o.dtype), _ptr(lse), _stream(stream)), "mx_attn_fwd_bf16_varlen")


def mx_attn_bwd_bf16_workspace_bytes(tokens, H) -> int:
    return lib().mx_attn_bwd_bf16_workspace_bytes(tokens, H)


def mx_attn_bwd_bf16(q, k, v, o, dout, lse, B, S, H, D, softmax_scale, causal, dq, dk, dv, workspace, stream=None):
    _check(lib().mx_attn_bwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), B, S, H, D,
                                  float(softmax_scale), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv),
                                  _dtype_code(dq.dtype), _ptr(workspace), workspace.numel(), _stream(stream)),
           "mx_attn_bwd_bf16")


def mx_attn_bwd_bf16_varlen(q, k, v, o, dout, lse, cu_seqlens, nseq, total_tokens, max_seqlen, H, D, softmax_scale,
                            causal, dq, dk, dv, workspace, stream=None):
    _check(lib().mx_attn_bwd_bf16_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(cu_seqlens),
                                         nseq, total_tokens, max_seqlen, H, D, float(softmax_scale),
                                         int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq.dtype),
                                         _ptr(workspace), workspace.numel(), _stream(stream)),
           "mx_attn_bwd_bf16_varlen")


def mx_attn_bwd_workspace_bytes(tokens, H, D) -> int:
    return lib().mx_attn_bwd_workspace_bytes(tokens, H, D)


def mx_attn_bwd_overflow(workspace, stream=None) -> bool:
    """True if the last backward on this workspace (None: this device's no-allocation scratch) left
    fp16's range (blocks on the stream)."""
    flag = ctypes.c_int(0)
    _check(lib().mx_attn_bwd_overflow(_ptr(workspace), ctypes.byref(flag), _stream(stream)), "mx_attn_bwd_overflow")
    return bool(flag.value)


def mx_attn_bwd(q_data, q_scale, k_data, k_scale, v_data, v_scale, do_data, do_scale, o, dout, lse, B, S, H, D,
                softmax_scale, causal, dq_scale_log2, dq, dk, dv, workspace, stream=None):
    _check(lib().mx_attn_bwd(_ptr(q_data), _ptr(q_scale), _ptr(k_data), _ptr(k_scale), _ptr(v_data), _ptr(v_scale),
                             _ptr(do_data), _ptr(do_scale), _ptr(o), _ptr(dout), _dtype_code(o.dtype), _ptr(lse),
                             B, S, H, D, float(softmax_scale), int(bool(causal)), int(dq_scale_log2), _ptr(dq),
                             _ptr(dk), _ptr(dv), _dtype_code(dq.dtype), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream)), "mx_attn_bwd")


def mx_attn_bwd_noalloc(q_data, q_scale, k_data, k_scale, v_data, v_scale, do_data, do_scale, o, dout, lse, B, S, H,
                        D, softmax_scale, causal, dq_scale_log2, dq, dk, dv, stream=None):
    _check(lib().mx_attn_bwd_noalloc(_ptr(q_data), _ptr(q_scale), _ptr(k_data), _ptr(k_scale), _ptr(v_data),
                                     _ptr(v_scale), _ptr(do_data), _ptr(do_scale), _ptr(o), _ptr(dout),
                                     _dtype_code(o.dtype), _ptr(lse), B, S, H, D, float(softmax_scale),
                                     int(bool(causal)), int(dq_scale_log2), _ptr(dq), _ptr(dk), _ptr(dv),
                                     _dtype_code(dq.dtype), _stream(stream)), "mx_attn_bwd_noalloc")


def mx_attn_bwd_varlen(q_data, q_scale, k_data, k_scale, v_data, v_scale, do_data, do_scale, o, dout, lse,
                       cu_seqlens, cu_scale_rows, nseq, total_tokens, max_seqlen, H, D, softmax_scale, causal,
                       dq_scale_log2, dq, dk, dv, workspace, stream=None):
    _check(lib().mx_attn_bwd_varlen(_ptr(q_data), _ptr(q_scale), _ptr(k_data), _ptr(k_scale), _ptr(v_data),
                                    _ptr(v_scale), _ptr(do_data), _ptr(do_scale), _ptr(o), _ptr(dout),
                                    _dtype_code(o.dtype), _ptr(lse), _ptr(cu_seqlens), _ptr(cu_scale_rows), nseq,
                                    total_tokens, max_seqlen, H, D, float(softmax_scale), int(bool(causal)),
                                    int(dq_scale_log2), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq.dtype),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream)), "mx_attn_bwd_varlen")


# ------------------------------------------------------------ allocation helpers
def scale_shape(layout: int, shape, total_scale_rows=None):
    """Scale tensor shape for a payload of ``shape`` ([B,S,H,D] or varlen [T,H,D])."""
    if len(shape) == 4:
        B, S, H, D = shape
        nb = (S + 31) // 32
        return {ROW32: (B, S, H, D // 32), COL32: (B, nb, H, D), SQ32: (B, nb, H, D // 32)}[layout]
    T, H, D = shape
    Tp = total_scale_rows
    return {ROW32: (Tp, H, D // 32), COL32: (Tp // 32, H, D), SQ32: (Tp // 32, H, D // 32)}[layout]


def alloc_quantized(shape, layouts, device, total_scale_rows=None):
    """Empty payload/scale tensors for every requested layout: {layout: (data, scale)}."""
    out = {}
    for lay in (ROW32, COL32, SQ32):
        if layouts & lay:
            data = torch.empty(shape, dtype=torch.uint8, device=device)
            scale = torch.empty(scale_shape(lay, shape, total_scale_rows), dtype=torch.uint8, device=device)
            out[lay] = (data, scale)
    return out


def quantize(x, layouts=ROW32 | COL32 | SQ32):
    """One-pass MX quantization of a [B, S, H, D] tensor; returns {layout: (data, scale)}."""
    B, S, H, D = x.shape
    out = alloc_quantized(x.shape, layouts, x.device)
    g = lambda lay, i: out[lay][i] if lay in out else None  # noqa: E731
    mx_quantize(x, B, S, H, D, layouts, g(ROW32, 0), g(ROW32, 1), g(COL32, 0), g(COL32, 1), g(SQ32, 0),
                g(SQ32, 1))
    return out


def rmsnorm_quantize(x, gamma, eps=1e-6, layouts=ROW32 | COL32 | SQ32):
    """Fused RMSNorm (over D, gain ``gamma`` fp32 [D]) + MX quantization of a [B, S, H, D]
    tensor; returns {layout: (data, scale)}."""
    B, S, H, D = x.shape
    out = alloc_quantized(x.shape, layouts, x.device)
    g = lambda lay, i: out[lay][i] if lay in out else None  # noqa: E731
    mx_rmsnorm_quantize(x, gamma, eps, B, S, H, D, layouts, g(ROW32, 0), g(ROW32, 1), g(COL32, 0), g(COL32, 1),
                        g(SQ32, 0), g(SQ32, 1))
    return out


def gemm_quantize(a, b, layouts=ROW32 | COL32 | SQ32, with_f32=False, fmt=E4M3):
    """C = A B^T from MX operands a = (data [M, K w/8], scale [M, K/32]) and b = (data [N, K w/8],
    scale [N, K/32]) in element format fmt; returns ({layout: (data [M, N], scale)}, C fp32 or None)."""
    M, K = a[0].shape[0], a[1].shape[1] * 32
    N = b[0].shape[0]
    dev = a[0].device
    shapes = {ROW32: (M, (N + 31) // 32), COL32: ((M + 31) // 32, N), SQ32: ((M + 31) // 32, (N + 31) // 32)}
    out = {lay: (torch.empty((M, N), dtype=torch.uint8, device=dev), torch.empty(shapes[lay], dtype=torch.uint8,
                                                                                   device=dev))
           for lay in (ROW32, COL32, SQ32) if layouts & lay}
    c32 = torch.empty((M, N), dtype=torch.float32, device=dev) if with_f32 else None
    g = lambda lay, i: out[lay][i] if lay in out else None  # noqa: E731
    mx_gemm_quantize(a[0], a[1], b[0], b[1], fmt, M, N, K, layouts, g(ROW32, 0), g(ROW32, 1), g(COL32, 0),
                     g(COL32, 1), g(SQ32, 0), g(SQ32, 1), c32)
    return out, c32


def mx_quantize_sq_fmt(x, B, S, H, D, fmt, row_data, col_data, scale, stream=None):
    _check(lib().mx_quantize_sq_fmt(_ptr(x), _dtype_code(x.dtype), B, S, H, D, fmt, _ptr(row_data), _ptr(col_data),
                                    _ptr(scale), _stream(stream)), "mx_quantize_sq_fmt")


def mx_quantize_sq_fmt_varlen(x, cu_seqlens, cu_scale_rows, nseq, total_tokens, total_scale_rows, H, D, fmt,
                              row_data, col_data, scale, stream=None):
    _check(lib().mx_quantize_sq_fmt_varlen(_ptr(x), _dtype_code(x.dtype), _ptr(cu_seqlens), _ptr(cu_scale_rows), nseq,
                                           total_tokens, total_scale_rows, H, D, fmt, _ptr(row_data), _ptr(col_data),
                                           _ptr(scale), _stream(stream)), "mx_quantize_sq_fmt_varlen")


def quantize_sq_fmt(x, fmt):
    """Square-block quantization of a [B, S, H, D] tensor in a small element format (E2M3, E3M2,
    E2M1).  Returns (row-packed data [B, S, H, D w/8], column-packed data [B, ceil(S/32), H, D, 32 w/8],
    scales [B, ceil(S/32), H, D/32])."""
    B, S, H, D = x.shape
    w, nb = ELEM_BITS[fmt], (S + 31) // 32
    row = torch.empty((B, S, H, D * w // 8), dtype=torch.uint8, device=x.device)
    col = torch.empty((B, nb, H, D, 32 * w // 8), dtype=torch.uint8, device=x.device)
    scale = torch.empty((B, nb, H, D // 32), dtype=torch.uint8, device=x.device)
    mx_quantize_sq_fmt(x, B, S, H, D, fmt, row, col, scale)
    return row, col, scale


def quantize_sq_fmt_varlen(x, cu_seqlens, cu_scale_rows, seqlens, fmt):
    """quantize_sq_fmt for a packed [T, H, D] tensor (jagged layout).  Returns (row-packed data
    [T, H, D w/8], column-packed data [Tp/32, H, D, 32 w/8], scales [Tp/32, H, D/32])."""
    T, H, D = x.shape
    Tp = padded_scale_rows(seqlens)
    w = ELEM_BITS[fmt]
    row = torch.empty((T, H, D * w // 8), dtype=torch.uint8, device=x.device)
    col = torch.empty((Tp // 32, H, D, 32 * w // 8), dtype=torch.uint8, device=x.device)
    scale = torch.empty((Tp // 32, H, D // 32), dtype=torch.uint8, device=x.device)
    mx_quantize_sq_fmt_varlen(x, cu_seqlens, cu_scale_rows, len(seqlens), T, Tp, H, D, fmt, row, col, scale)
    return row, col, scale


def quantize_rows(x, fmt=E4M3):
    """MX quantization of a [rows, K] operand along K in element format fmt.
    Returns (packed data [rows, K w/8], scales [rows, K/32])."""
    rows, K = x.shape
    data = torch.empty((rows, K * ELEM_BITS[fmt] // 8), dtype=torch.uint8, device=x.device)
    scale = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    mx_quantize_rows(x, rows, K, fmt, data, scale)
    return data, scale


def padded_scale_rows(seqlens) -> int:
    return int(sum((int(L) + 127) // 128 * 128 for L in seqlens))


def quantize_varlen(x, cu_seqlens, seqlens, layouts=ROW32 | COL32 | SQ32):
    """MX quantization of a packed [T, H, D] tensor; returns ({layout: (data, scale)}, cu_scale_rows)."""
    T, H, D = x.shape
    nseq = len(seqlens)
    Tp = padded_scale_rows(seqlens)
    csr = torch.empty(nseq + 1, dtype=torch.int32, device=x.device)
    mx_varlen_scale_offsets(cu_seqlens, nseq, csr)
    out = alloc_quantized(x.shape, layouts, x.device, Tp)
    g = lambda lay, i: out[lay][i] if lay in out else None  # noqa: E731
    mx_quantize_varlen(x, cu_seqlens, csr, nseq, T, Tp, H, D, layouts, g(ROW32, 0), g(ROW32, 1), g(COL32, 0),
                       g(COL32, 1), g(SQ32, 0), g(SQ32, 1))
    return out, csr


def quantize_rows_varlen(x, cu_seqlens, cu_scale_rows, seqlens, fmt=E4M3):
    """Row quantization (element format fmt) of a packed [T, H, D] tensor in the jagged layout
    (mx_quantize_rows_varlen: scale rows at the 128-aligned per-sequence offsets, pad rows zero).
    Returns (packed data [T, H, D w/8], scales [Tp, H, D/32])."""
    T, H, D = x.shape
    Tp = padded_scale_rows(seqlens)
    data = torch.empty((T, H, D * ELEM_BITS[fmt] // 8), dtype=torch.uint8, device=x.device)
    scale = torch.empty((Tp, H, D // 32), dtype=torch.uint8, device=x.device)
    mx_quantize_rows_varlen(x, cu_seqlens, cu_scale_rows, len(seqlens), T, Tp, H, D, fmt, data, scale)
    return data, scale


def rmsnorm_quantize_varlen(x, gamma, cu_seqlens, seqlens, eps=1e-6, layouts=ROW32 | COL32 | SQ32):
    """Fused RMSNorm + MX quantization of a packed [T, H, D] tensor; returns
    ({layout: (data, scale)}, cu_scale_rows)."""
    T, H, D = x.shape
    nseq = len(seqlens)
    Tp = padded_scale_rows(seqlens)
    csr = torch.empty(nseq + 1, dtype=torch.int32, device=x.device)
    mx_varlen_scale_offsets(cu_seqlens, nseq, csr)
    out = alloc_quantized(x.shape, layouts, x.device, Tp)
    g = lambda lay, i: out[lay][i] if lay in out else None  # noqa: E731
    mx_rmsnorm_quantize_varlen(x, gamma, eps, cu_seqlens, csr, nseq, T, Tp, H, D, layouts, g(ROW32, 0),
                               g(ROW32, 1), g(COL32, 0), g(COL32, 1), g(SQ32, 0), g(SQ32, 1))
    return out, csr


def attn_fwd(q, k, v, softmax_scale, causal, out_dtype=torch.bfloat16, with_lse=True):
    """q, k: (data, scale) ROW32; v: (data, scale) COL32.  Returns (O, LSE)."""
    B, S, H, D = q[0].shape
    o = torch.empty((B, S, H, D), dtype=out_dtype, device=q[0].device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q[0].device) if with_lse else None
    mx_attn_fwd(q[0], q[1], k[0], k[1], v[0], v[1], B, S, H, D, softmax_scale, causal, o, lse)
    return o, lse


def attn_fwd_fmt(q, k, v, shape, softmax_scale, causal, qk_format, out_dtype=torch.bfloat16, with_lse=True):
    """q, k: (packed data, ROW32 scales) in element format qk_format, as quantize_rows gives them for
    the [B*S*H, D] view; v: (data, scale) COL32; shape = (B, S, H, D).  Returns (O, LSE)."""
    B, S, H, D = shape
    o = torch.empty((B, S, H, D), dtype=out_dtype, device=v[0].device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=v[0].device) if with_lse else None
    mx_attn_fwd_fmt(q[0], q[1], k[0], k[1], v[0], v[1], B, S, H, D, softmax_scale, causal, qk_format, o, lse)
    return o, lse


def attn_fwd_bf16(q, k, v, softmax_scale, causal, out_dtype=torch.bfloat16, with_lse=True):
    """BF16 attention forward: q, k, v bfloat16 [B, S, H, D].  Returns (O, LSE)."""
    B, S, H, D = q.shape
    o = torch.empty((B, S, H, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if with_lse else None
    mx_attn_fwd_bf16(q, k, v, B, S, H, D, softmax_scale, causal, o, lse)
    return o, lse


def attn_fwd_bf16_varlen(q, k, v, cu_seqlens, seqlens, softmax_scale, causal, out_dtype=torch.bfloat16,
                         with_lse=True):
    T, H, D = q.shape
    o = torch.empty((T, H, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if with_lse else None
    mx_attn_fwd_bf16_varlen(q, k, v, cu_seqlens, len(seqlens), T, max(seqlens), H, D, softmax_scale, causal, o, lse)
    return o, lse


def attn_bwd_bf16(q, k, v, o, dout, lse, softmax_scale, causal, grad_dtype=torch.bfloat16):
    """BF16 attention backward: q, k, v, o, dout bfloat16 [B, S, H, D], lse [B, H, S].
    Returns (dQ, dK, dV)."""
    B, S, H, D = q.shape
    dq, dk, dv = (torch.empty((B, S, H, D), dtype=grad_dtype, device=q.device) for _ in range(3))
    ws = torch.empty(mx_attn_bwd_bf16_workspace_bytes(B * S, H), dtype=torch.uint8, device=q.device)
    mx_attn_bwd_bf16(q, k, v, o, dout, lse, B, S, H, D, softmax_scale, causal, dq, dk, dv, ws)
    return dq, dk, dv


def attn_bwd_bf16_varlen(q, k, v, o, dout, lse, cu_seqlens, seqlens, softmax_scale, causal,
                         grad_dtype=torch.bfloat16):
    T, H, D = q.shape
    dq, dk, dv = (torch.empty((T, H, D), dtype=grad_dtype, device=q.device) for _ in range(3))
    ws = torch.empty(mx_attn_bwd_bf16_workspace_bytes(T, H), dtype=torch.uint8, device=q.device)
    mx_attn_bwd_bf16_varlen(q, k, v, o, dout, lse, cu_seqlens, len(seqlens), T, max(seqlens), H, D, softmax_scale,
                            causal, dq, dk, dv, ws)
    return dq, dk, dv


def attn_fwd_varlen(q, k, v, cu_seqlens, cu_scale_rows, seqlens, softmax_scale, causal,
                    out_dtype=torch.bfloat16, with_lse=True):
    T, H, D = q[0].shape
    o = torch.empty((T, H, D), dtype=out_dtype, device=q[0].device)
    lse = torch.empty((H, T), dtype=torch.float32, device=q[0].device) if with_lse else None
    mx_attn_fwd_varlen(q[0], q[1], k[0], k[1], v[0], v[1], cu_seqlens, cu_scale_rows, len(seqlens), T,
                       max(seqlens), H, D, softmax_scale, causal, o, lse)
    return o, lse


def attn_fwd_fmt_varlen(q, k, v, cu_seqlens, cu_scale_rows, seqlens, softmax_scale, causal, qk_format,
                        out_dtype=torch.bfloat16, with_lse=True):
    """q, k: (data, scales) from quantize_rows_varlen in element format qk_format; v: (data, scale)
    COL32 from quantize_varlen.  Returns (O [T, H, D], LSE [H, T])."""
    T, H = q[0].shape[:2]
    D = q[1].shape[2] * 32
    o = torch.empty((T, H, D), dtype=out_dtype, device=q[0].device)
    lse = torch.empty((H, T), dtype=torch.float32, device=q[0].device) if with_lse else None
    mx_attn_fwd_fmt_varlen(q[0], q[1], k[0], k[1], v[0], v[1], cu_seqlens, cu_scale_rows, len(seqlens), T,
                           max(seqlens), H, D, softmax_scale, causal, qk_format, o, lse)
    return o, lse


def attn_bwd(q, k, v, do, o, dout, lse, softmax_scale, causal, dq_scale_log2, grad_dtype=torch.bfloat16,
             with_overflow=False):
    """q, k, do: (data, scale) SQ32; v: (data, scale) ROW32; o, dout: [B,S,H,D]; lse [B,H,S].
    Returns (dQ, dK, dV), plus the fp16 range flag (mx_attn_bwd_overflow) with with_overflow=True."""
    B, S, H, D = q[0].shape
    dev = q[0].device
    dq, dk, dv = (torch.empty((B, S, H, D), dtype=grad_dtype, device=dev) for _ in range(3))
    ws = torch.empty(mx_attn_bwd_workspace_bytes(B * S, H, D), dtype=torch.uint8, device=dev)
    mx_attn_bwd(q[0], q[1], k[0], k[1], v[0], v[1], do[0], do[1], o, dout, lse, B, S, H, D, softmax_scale, causal,
                dq_scale_log2, dq, dk, dv, ws)
    if with_overflow:
        return dq, dk, dv, mx_attn_bwd_overflow(ws)
    return dq, dk, dv


def mx_attn_bwd_fmt(q_row, q_col, q_scale, k_row, k_col, k_scale, v_data, v_scale, do_data, do_scale, o, dout, lse,
                    B, S, H, D, softmax_scale, causal, dq_scale_log2, qk_format, dq, dk, dv, workspace, stream=None):
    _check(lib().mx_attn_bwd_fmt(_ptr(q_row), _ptr(q_col), _ptr(q_scale), _ptr(k_row), _ptr(k_col), _ptr(k_scale),
                                 _ptr(v_data), _ptr(v_scale), _ptr(do_data), _ptr(do_scale), _ptr(o), _ptr(dout),
                                 _dtype_code(o.dtype), _ptr(lse), B, S, H, D, float(softmax_scale), int(bool(causal)),
                                 int(dq_scale_log2), int(qk_format), _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq.dtype),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream)),
           "mx_attn_bwd_fmt")


def mx_attn_bwd_fmt_varlen(q_row, q_col, q_scale, k_row, k_col, k_scale, v_data, v_scale, do_data, do_scale, o, dout,
                           lse, cu_seqlens, cu_scale_rows, nseq, total_tokens, max_seqlen, H, D, softmax_scale, causal,
                           dq_scale_log2, qk_format, dq, dk, dv, workspace, stream=None):
    _check(lib().mx_attn_bwd_fmt_varlen(_ptr(q_row), _ptr(q_col), _ptr(q_scale), _ptr(k_row), _ptr(k_col),
                                        _ptr(k_scale), _ptr(v_data), _ptr(v_scale), _ptr(do_data), _ptr(do_scale),
                                        _ptr(o), _ptr(dout), _dtype_code(o.dtype), _ptr(lse), _ptr(cu_seqlens),
                                        _ptr(cu_scale_rows), nseq, total_tokens, max_seqlen, H, D,
                                        float(softmax_scale), int(bool(causal)), int(dq_scale_log2), int(qk_format),
                                        _ptr(dq), _ptr(dk), _ptr(dv), _dtype_code(dq.dtype), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)),
           "mx_attn_bwd_fmt_varlen")


def attn_bwd_fmt(q, k, v, do, o, dout, lse, softmax_scale, causal, dq_scale_log2, qk_format,
                 grad_dtype=torch.bfloat16, with_overflow=False):
    """q, k: (row-packed, column-packed, scales) from quantize_sq_fmt in element format qk_format;
    v: (data, scale) ROW32; do: (data, scale) SQ32; o, dout: [B,S,H,D]; lse [B,H,S].
    Returns (dQ, dK, dV), plus the fp16 range flag with with_overflow=True."""
    B, S, H, D = o.shape
    dev = o.device
    dq, dk, dv = (torch.empty((B, S, H, D), dtype=grad_dtype, device=dev) for _ in range(3))
    ws = torch.empty(mx_attn_bwd_workspace_bytes(B * S, H, D), dtype=torch.uint8, device=dev)
    mx_attn_bwd_fmt(q[0], q[1], q[2], k[0], k[1], k[2], v[0], v[1], do[0], do[1], o, dout, lse, B, S, H, D,
                    softmax_scale, causal, dq_scale_log2, qk_format, dq, dk, dv, ws)
    if with_overflow:
        return dq, dk, dv, mx_attn_bwd_overflow(ws)
    return dq, dk, dv


def attn_bwd_fmt_varlen(q, k, v, do, o, dout, lse, cu_seqlens, cu_scale_rows, seqlens, softmax_scale, causal,
                        dq_scale_log2, qk_format, grad_dtype=torch.bfloat16, with_overflow=False):
    """attn_bwd_fmt over packed sequences (q, k from quantize_sq_fmt_varlen)."""
    T, H, D = o.shape
    dev = o.device
    dq, dk, dv = (torch.empty((T, H, D), dtype=grad_dtype, device=dev) for _ in range(3))
    ws = torch.empty(mx_attn_bwd_workspace_bytes(T, H, D), dtype=torch.uint8, device=dev)
    mx_attn_bwd_fmt_varlen(q[0], q[1], q[2], k[0], k[1], k[2], v[0], v[1], do[0], do[1], o, dout, lse, cu_seqlens,
                           cu_scale_rows, len(seqlens), T, max(seqlens), H, D, softmax_scale, causal, dq_scale_log2,
                           qk_format, dq, dk, dv, ws)
    if with_overflow:
        return dq, dk, dv, mx_attn_bwd_overflow(ws)
    return dq, dk, dv


def attn_bwd_varlen(q, k, v, do, o, dout, lse, cu_seqlens, cu_scale_rows, seqlens, softmax_scale, causal,
                    dq_scale_log2, grad_dtype=torch.bfloat16, with_overflow=False):
    T, H, D = q[0].shape
    dev = q[0].device
    dq, dk, dv = (torch.empty((T, H, D), dtype=grad_dtype, device=dev) for _ in range(3))
    ws = torch.empty(mx_attn_bwd_workspace_bytes(T, H, D), dtype=torch.uint8, device=dev)
    mx_attn_bwd_varlen(q[0], q[1], k[0], k[1], v[0], v[1], do[0], do[1], o, dout, lse, cu_seqlens, cu_scale_rows,
                       len(seqlens), T, max(seqlens), H, D, softmax_scale, causal, dq_scale_log2, dq, dk, dv, ws)
    if with_overflow:
        return dq, dk, dv, mx_attn_bwd_overflow(ws)
    return dq, dk, dv
