/*
 * mxfa.h -- MXFP8 block-scaled attention for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels: MX quantization, the fused MXFP8
 * attention forward, and the fused MXFP8 attention backward, each with a
 * fixed-length and a jagged (varlen) form; the fused producers (RMSNorm +
 * quantize, GEMM + quantize) and the BF16 attention baseline.
 *
 * Pages cited (by title):
 *   [News]  "Low Precision Flash Attention 4: End-to-End Block-Scaled
 *           Attention for Blackwell"
 *   [Blog]  "Low-Precision FlashAttention-4: End-to-End Block-Scaled
 *           Attention for NVIDIA Blackwell"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * MX format ([Blog], "Understanding OCP MXFP8 Microscaling on Blackwell"):
 *   blocks of 32 elements share one E8M0 scale byte k (value 2^(k-127));
 *   each element is one OCP E4M3FN byte (bias 7, max 448, 0x7F/0xFF NaN).
 *   The scale of a block is k = clamp(floor(log2(amax)) - 8 + 127, 0, 254)
 *   (OCP MX rule; k = 0 for an all-zero block); elements are encoded as
 *   E4M3(x * 2^(127-k)) rounded to nearest even and saturated to +-448.
 *
 * Tensors are dense and row-major.  Fixed-length activations are
 *   [B, S, H, D] (D contiguous), the shape of the pages' attention call
 *   ([Blog], "PyTorch Integration & Implementation Example").  Jagged
 *   activations are packed [T, H, D]; sequence s occupies tokens
 *   cu_seqlens[s] .. cu_seqlens[s+1]-1.
 *
 * An MX tensor is a payload (uint8, same shape and index as the source
 * element: the FP8 data stays at its unpadded position, [News],
 * contributions paragraph) plus a scale tensor in one of three layouts:
 *   MX_ROW32  blocks of 32 consecutive features of one token.
 *             scales [B, S, H, D/32]        (varlen: [Tpad, H, D/32])
 *   MX_COL32  blocks of 32 consecutive tokens of one feature (blocked from
 *             the sequence start; the last block may be short).
 *             scales [B, ceil(S/32), H, D]  (varlen: [Tpad/32, H, D])
 *   MX_SQ32   square blocks of 32 tokens x 32 features.  The payload is the
 *             same whichever axis is contracted ([News], forward/backward
 *             paragraph).
 *             scales [B, ceil(S/32), H, D/32] (varlen: [Tpad/32, H, D/32])
 * Varlen scale tensors are padded per sequence to 128-row boundaries
 * ([News], contributions paragraph: only the scales are scattered and
 * padded, to 128-aligned addresses): sequence s owns scale rows
 * cu_scale_rows[s] .. cu_scale_rows[s+1]-1 (ROW32) or
 * cu_scale_rows[s]/32 .. (COL32, SQ32), where cu_scale_rows is the prefix
 * sum of roundup(L_s, 128) (see mx_varlen_scale_offsets).  Pad slots are
 * written as 0.
 *
 * Memory and streams: every pointer argument is device memory owned by the
 * caller unless stated otherwise; the library never allocates or frees and
 * keeps no pointer after the call returns (kernels queued on `stream` still
 * use them).  Every call is asynchronous on `stream` (0 = the null stream)
 * and does not synchronise the host.  Device pointers must be 16-byte
 * aligned.  The library holds no state and may be called from any thread.
 *
 * Errors: arguments are validated on the host before anything is launched;
 * an invalid call returns MX_EINVAL (or MX_EWORKSPACE) and launches nothing.
 * A device that is not gfx950 gives MX_EUNSUPPORTED; a failed launch gives
 * MX_EHIP.  Non-finite inputs are outside the contract: results are then
 * unspecified, but no call faults.  Integer device inputs (cu_seqlens,
 * cu_scale_rows) must be consistent with the host sizes passed beside them;
 * this is the caller's responsibility (the device does not validate them).
 * Size limits (MX_EINVAL beyond them): at most 2^40 elements per tensor,
 * 2^31 - 1 tokens per call (B * S or total_tokens) and 2^16 heads.
 */
#ifndef MXFA_H
#define MXFA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MXFA_ABI_VERSION 1

typedef enum {
  MX_OK = 0,
  MX_EINVAL = 1,        /* bad argument (shape, pointer, alignment, dtype) */
  MX_EUNSUPPORTED = 2,  /* device is not gfx950, or an unsupported combination */
  MX_EHIP = 3,          /* a HIP runtime call or kernel launch failed */
  MX_EWORKSPACE = 4     /* workspace pointer null or too small */
} mx_status;

typedef enum { MX_F32 = 0, MX_BF16 = 1, MX_F16 = 2 } mx_dtype;

enum { MX_ROW32 = 1, MX_COL32 = 2, MX_SQ32 = 4 };

/* Element formats of MX payloads, numbered as the block-scaled matrix
 * instruction's format fields: MXFP8 E4M3, MXFP6 E2M3 and E3M2, MXFP4 E2M1
 * ([News], paragraph on the block-scaled MMA instructions; element
 * definitions of OCP MX v1.0: no Inf/NaN in the 6- and 4-bit formats,
 * round to nearest even, saturating).  A w-bit payload row is a
 * little-endian bitstream: element j at bits [w j, w j + w). */
typedef enum { MX_E4M3 = 0, MX_E2M3 = 2, MX_E3M2 = 3, MX_E2M1 = 4 } mx_elem;

/* ABI version (MXFA_ABI_VERSION) and a static string for a status code. */
int mx_abi_version(void);
const char* mx_status_str(mx_status s);

/*
 * mx_quantize -- MX quantization of a [B, S, H, D] tensor in one pass.
 * Defines: the MX block format of [Blog], "Understanding OCP MXFP8
 * Microscaling on Blackwell", with the dual/multiple scale layouts written
 * in one pass of [News], contributions paragraph.
 *   x          input, x_dtype MX_BF16 or MX_F32, [B, S, H, D]
 *   D          64 or 128; S >= 0 (any value; COL32/SQ32 tail blocks short)
 *   layouts    nonzero bitmask of MX_ROW32 | MX_COL32 | MX_SQ32
 *   *_data     payload [B, S, H, D] uint8 for each requested layout
 *   *_scale    scales in that layout's shape (see above)
 * Buffers of layouts not requested are ignored and may be NULL.
 */
mx_status mx_quantize(const void* x, mx_dtype x_dtype, int B, int S, int H, int D,
                      unsigned layouts,
                      uint8_t* row32_data, uint8_t* row32_scale,
                      uint8_t* col32_data, uint8_t* col32_scale,
                      uint8_t* sq32_data, uint8_t* sq32_scale,
                      hipStream_t stream);

/*
 * mx_varlen_scale_offsets -- cu_scale_rows[s] = sum_{u<s} roundup(L_u, 128)
 * from cu_seqlens (both device int32 arrays of nseq+1 entries).
 * Defines: the 128-aligned scale placement of jagged tensors, [News],
 * contributions paragraph.  One tiny kernel; nseq >= 1.
 */
mx_status mx_varlen_scale_offsets(const int32_t* cu_seqlens, int nseq, int32_t* cu_scale_rows,
                                  hipStream_t stream);

/*
 * mx_quantize_varlen -- mx_quantize for a packed [T, H, D] tensor.
 * Defines: the jagged layout of [News], contributions paragraph (FP8 payload
 * at its unpadded packed position, scales at padded 128-aligned per-sequence
 * offsets), with mx_quantize's blocks ([Blog], "Understanding OCP MXFP8
 * Microscaling on Blackwell"; square blocks: [News], forward/backward
 * paragraph).
 *   x                           [T, H, D] in x_dtype (MX_BF16 or MX_F32)
 *   cu_seqlens, cu_scale_rows   device int32 [nseq+1] (mx_varlen_scale_offsets)
 *   total_tokens                T = cu_seqlens[nseq] (host int)
 *   total_scale_rows            Tpad = cu_scale_rows[nseq] (a multiple of 128)
 *   outputs                     payload [T, H, D]; ROW32 scales [Tpad, H, D/32],
 *                               COL32 [Tpad/32, H, D], SQ32 [Tpad/32, H, D/32]
 * Blocks along tokens start at each sequence's first token (short tail
 * blocks); pad scale slots are written as 0.  Errors: as mx_quantize, and
 * MX_EINVAL for nseq < 1, null offset arrays or negative totals; T = 0: MX_OK.
 */
mx_status mx_quantize_varlen(const void* x, mx_dtype x_dtype,
                             const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq,
                             int total_tokens, int total_scale_rows, int H, int D,
                             unsigned layouts,
                             uint8_t* row32_data, uint8_t* row32_scale,
                             uint8_t* col32_data, uint8_t* col32_scale,
                             uint8_t* sq32_data, uint8_t* sq32_scale,
                             hipStream_t stream);

/*
 * mx_rmsnorm_quantize -- fused RMSNorm + MX quantization (one read of x).
 * Defines: [News], contributions paragraph (fused RMSNorm + Quantize
 * producers emitting FP8 with several scale layouts in one pass).  The
 * pages give no formula; this library's reading (the usual RMSNorm, per
 * (token, head) row over D, as for normalized query and key heads):
 *   rstd = fl32(1 / sqrt(sum_d x_d^2 / D + eps))   (sum, divide, sqrt and
 *          reciprocal in fp64; the squares of bf16 / fp32 inputs are exact)
 *   y_d  = fl32(fl32(x_d * rstd) * gamma_d)
 * then y is quantized exactly as mx_quantize quantizes x.
 *   gamma   device fp32 [D], 4-byte aligned (read only)
 *   eps     finite, >= 0
 * Everything else (layouts, shapes, outputs, errors) as mx_quantize;
 * MX_EINVAL also for a null or misaligned gamma or a bad eps.
 */
mx_status mx_rmsnorm_quantize(const void* x, mx_dtype x_dtype, const float* gamma, float eps,
                              int B, int S, int H, int D, unsigned layouts,
                              uint8_t* row32_data, uint8_t* row32_scale,
                              uint8_t* col32_data, uint8_t* col32_scale,
                              uint8_t* sq32_data, uint8_t* sq32_scale,
                              hipStream_t stream);

/*
 * mx_rmsnorm_quantize_varlen -- mx_rmsnorm_quantize for a packed [T, H, D]
 * tensor; the sequence arguments as mx_quantize_varlen.
 */
mx_status mx_rmsnorm_quantize_varlen(const void* x, mx_dtype x_dtype, const float* gamma, float eps,
                                     const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq,
                                     int total_tokens, int total_scale_rows, int H, int D,
                                     unsigned layouts,
                                     uint8_t* row32_data, uint8_t* row32_scale,
                                     uint8_t* col32_data, uint8_t* col32_scale,
                                     uint8_t* sq32_data, uint8_t* sq32_scale,
                                     hipStream_t stream);

/*
 * mx_quantize_rows -- MX quantization of a GEMM operand in any element format:
 * blocks of 32 along each row of x [rows, K] (the contraction axis), E8M0
 * scale clamp(floor(log2 amax) - emax + 127, 0, 254) with emax = 8 (E4M3),
 * 2 (E2M3, E2M1) or 4 (E3M2), elements RNE-encoded and saturated.
 *   x       [rows, K] in x_dtype (MX_BF16 or MX_F32), 16-byte aligned
 *   K       a positive multiple of 32
 *   data    [rows, K * w / 8] bytes, w = 8, 6, 4 bits (16-byte aligned)
 *   scale   [rows, K / 32] E8M0 bytes
 * For E4M3 this equals mx_quantize's ROW32 output of an [rows, 1, K/D, D]
 * tensor.  Errors: MX_EINVAL for a bad shape, format, dtype or alignment;
 * rows = 0: MX_OK.  Ownership: caller's buffers.
 */
mx_status mx_quantize_rows(const void* x, mx_dtype x_dtype, int rows, int K, mx_elem format,
                           uint8_t* data, uint8_t* scale, hipStream_t stream);

/*
 * mx_quantize_rows_varlen -- mx_quantize_rows for a packed [T, H, K] tensor
 * in the jagged layout: payload rows [T, H, K*w/8] at their packed token
 * positions, scale rows [Tpad, H, K/32] at the 128-aligned per-sequence
 * offsets ([News], contributions paragraph), pad rows written as 0.
 * Defines: as mx_quantize_rows (the MXFP6 / MXFP4 operands of [News],
 * paragraph on the block-scaled MMA's formats), with the placement above.
 *   x              [T, H, K] in x_dtype (MX_BF16 or MX_F32), 16-byte aligned
 *   cu_seqlens, cu_scale_rows   device int32 [nseq+1] (mx_varlen_scale_offsets)
 *   total_tokens, total_scale_rows   T and Tpad (host ints)
 *   data, scale    outputs as above
 * Errors: as mx_quantize_rows, and MX_EINVAL for nseq < 1, null offset arrays
 * or negative totals; T = 0: MX_OK.  Ownership: caller's buffers.
 */
mx_status mx_quantize_rows_varlen(const void* x, mx_dtype x_dtype, const int32_t* cu_seqlens,
                                  const int32_t* cu_scale_rows, int nseq, int total_tokens,
                                  int total_scale_rows, int H, int K, mx_elem format,
                                  uint8_t* data, uint8_t* scale, hipStream_t stream);

/*
 * mx_quantize_sq_fmt -- square [32 tokens x 32 features] blocks of a [B, S, H, D]
 * tensor in a small element format, for the backward's Q and K with MXFP6 /
 * MXFP4 payloads (mx_attn_bwd_fmt).
 * Defines: [News], forward/backward paragraph (Q, K in square [32, 32] blocks
 * so one set of codes serves both orientations) with the element formats of
 * [News]' paragraph on the block-scaled MMA (OCP MX E2M3, E3M2, E2M1); the E8M0
 * scale of a block is clamp(floor(log2 amax) - emax + 127, 0, 254), emax 2, 4, 2.
 * Blocks start at token 0 and feature 0; a short tail block holds the rest.
 *   x          [B, S, H, D] in x_dtype (MX_BF16 or MX_F32), 16-byte aligned; D = 64 or 128
 *   format     MX_E2M3, MX_E3M2 or MX_E2M1
 *   row_data   [B, S, H, D*w/8] bytes: each token row along D, packed as the
 *              matrix instruction reads it (element j at bits [w j, w j + w))
 *   col_data   [B, ceil(S/32), H, D, 32*w/8] bytes: for each block row and
 *              feature, that feature's 32 tokens packed the same way (tokens
 *              past S as code 0) -- the same codes read across the rows
 *   scale      [B, ceil(S/32), H, D/32] E8M0 bytes (the SQ32 scale layout)
 * Errors: MX_EINVAL for a bad shape, format, dtype, alignment or null
 * output; B*S = 0: MX_OK.  Ownership: caller's buffers.
 */
mx_status mx_quantize_sq_fmt(const void* x, mx_dtype x_dtype, int B, int S, int H, int D, mx_elem format,
                             uint8_t* row_data, uint8_t* col_data, uint8_t* scale, hipStream_t stream);

/*
 * mx_quantize_sq_fmt_varlen -- mx_quantize_sq_fmt for a packed [T, H, D] tensor
 * in the jagged layout ([News], contributions paragraph): row_data [T, H, D*w/8]
 * at the packed token positions; col_data [Tpad/32, H, D, 32*w/8] and scale
 * [Tpad/32, H, D/32] at the 128-aligned per-sequence block rows, pad rows
 * written as 0.  Sequence arguments as mx_quantize_rows_varlen.
 * Errors: as mx_quantize_sq_fmt, and as mx_quantize_rows_varlen for the
 * sequence arguments; T = 0: MX_OK.  Ownership: caller's buffers.
 */
mx_status mx_quantize_sq_fmt_varlen(const void* x, mx_dtype x_dtype, const int32_t* cu_seqlens,
                                    const int32_t* cu_scale_rows, int nseq, int total_tokens,
                                    int total_scale_rows, int H, int D, mx_elem format,
                                    uint8_t* row_data, uint8_t* col_data, uint8_t* scale, hipStream_t stream);

/*
 * mx_gemm_quantize -- MX GEMM with a quantizing epilogue: C = A B^T.
 * Defines: [News], contributions paragraph (fused GEMM + Quantize producers
 * emitting FP8 with several scale layouts in one pass); the block-scaled
 * GEMM itself as in [Blog], "1. End-to-End Block-Scaled GEMM Fusion".
 *   a_data, a_scale  A [M, K] payload in ab_format (packed rows of K*w/8
 *                    bytes, as mx_quantize_rows writes), ROW32 scales [M, K/32]
 *   b_data, b_scale  B [N, K] likewise
 *   ab_format        element format of A and B: MX_E4M3, MX_E2M3, MX_E3M2 or
 *                    MX_E2M1 (the matrix instruction's format fields; the
 *                    6- and 4-bit formats are the pages' MXFP6 / MXFP4)
 *                    (B is the [out, in] weight; C[m, n] = sum_k A[m,k] B[n,k])
 *   C is accumulated in fp32 by the block-scaled matrix instruction, then
 *   quantized to MXFP8 in the requested layouts (0 allowed when c_f32 is
 *   given), blocks aligned at row and column 0, short tail blocks at the
 *   edges, encoding as mx_quantize:
 *     ROW32  payload [M, N], scales [M, ceil(N/32)]   (32 columns per block)
 *     COL32  payload [M, N], scales [ceil(M/32), N]   (32 rows per block)
 *     SQ32   payload [M, N], scales [ceil(M/32), ceil(N/32)]
 *   c_f32  optional fp32 copy of C [M, N] (may be NULL)
 * Requirements: K a positive multiple of 64 and at most 2^20, N a multiple of 16, every
 * pointer 16-byte aligned.  MX_EINVAL otherwise; M = 0 or N = 0: MX_OK.
 * Ownership: all buffers belong to the caller; nothing is allocated.
 */
mx_status mx_gemm_quantize(const uint8_t* a_data, const uint8_t* a_scale,
                           const uint8_t* b_data, const uint8_t* b_scale, mx_elem ab_format,
                           int M, int N, int K, unsigned layouts,
                           uint8_t* c_row32_data, uint8_t* c_row32_scale,
                           uint8_t* c_col32_data, uint8_t* c_col32_scale,
                           uint8_t* c_sq32_data, uint8_t* c_sq32_scale,
                           float* c_f32, hipStream_t stream);

/*
 * mx_attn_fwd -- fused MXFP8 attention forward.
 * Defines: [Blog], "1. End-to-End Block-Scaled GEMM Fusion" (S = Q K^T and
 * P V both on block-scaled operands, nothing written to HBM in between) and
 * "2. Synchronized Online Softmax with Dynamic Scaling" (FP32 online
 * softmax, logits scaled by softmax_scale); [News], forward/backward
 * paragraph (P converted to MXFP8, its scales taken from the max the
 * softmax already computed).
 * Computation per (b, h), with c = fl32(softmax_scale * log2(e)):
 *   S = Q^ K^T (Q^, K^ ROW32; the scaled MFMA's fp32 result, within the stated product
 *   error bound of the exact sum -- see the oracle's reading of the matrix unit);
 *   M_i = ceil(fl32(max_j S_ij * c)) (an integer frame);
 *   p_ij = 2^(S_ij c - M_i) (fp32), l_i = sum_j p_ij;
 *   P^ = MX(p) in blocks of 32 keys per query (aligned at key 0);
 *   O = (P^ V^) / l  with V^ in COL32;  LSE_i = ln2 * (M_i + log2 l_i).
 *   q_data, q_scale, k_data, k_scale   ROW32 payload + scales
 *   v_data, v_scale                    COL32 payload + scales
 *   D 64 or 128; S >= 1; causal keeps keys j <= i
 *   o        [B, S, H, D], o_dtype MX_BF16 or MX_F32 (rounded to nearest even)
 *   lse      [B, H, S] fp32, natural log; may be NULL
 */
mx_status mx_attn_fwd(const uint8_t* q_data, const uint8_t* q_scale,
                      const uint8_t* k_data, const uint8_t* k_scale,
                      const uint8_t* v_data, const uint8_t* v_scale,
                      int B, int S, int H, int D, float softmax_scale, int causal,
                      void* o, mx_dtype o_dtype, float* lse, hipStream_t stream);

/*
 * mx_attn_fwd_varlen -- mx_attn_fwd over packed sequences.
 * Defines: [News], contributions paragraph (a jagged attention whose FP8
 * payload stays unpadded while its scales sit at 128-aligned per-sequence
 * offsets), applied to mx_attn_fwd's computation per sequence.
 *   q_*, k_*   [T, H, D] payloads, ROW32 scales [Tpad, H, D/32]
 *   v_*        [T, H, D] payload, COL32 scales [Tpad/32, H, D]
 *   cu_seqlens, cu_scale_rows   device int32 [nseq+1] (as mx_quantize_varlen)
 *   total_tokens T; max_seqlen bounds every L_s (host ints)
 *   o          [T, H, D]; lse [H, T] fp32 (may be null)
 * Causality is within each sequence; empty sequences are allowed.  Errors:
 * as mx_attn_fwd, and MX_EINVAL for nseq < 1 or null offset arrays; T = 0 or
 * max_seqlen = 0: MX_OK.  Ownership: caller's buffers.
 */
mx_status mx_attn_fwd_varlen(const uint8_t* q_data, const uint8_t* q_scale,
                             const uint8_t* k_data, const uint8_t* k_scale,
                             const uint8_t* v_data, const uint8_t* v_scale,
                             const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq,
                             int total_tokens, int max_seqlen, int H, int D,
                             float softmax_scale, int causal,
                             void* o, mx_dtype o_dtype, float* lse, hipStream_t stream);

/*
 * mx_attn_fwd_fmt -- mx_attn_fwd with Q and K in MXFP6 or MXFP4.
 * Defines: [News], paragraph on Blackwell's block-scaled MMA instructions (MXFP8,
 * MXFP6 and MXFP4 operands of the same block-scaled product), applied to the
 * forward's S = Q^ K^T of [Blog], "1. End-to-End Block-Scaled GEMM Fusion".
 * Reading (the pages define neither format): the OCP MX v1.0 elements, as for
 * mx_quantize_rows; P and V stay MXFP8 and every later step is mx_attn_fwd's.
 *   qk_format   MX_E4M3 (identical to mx_attn_fwd), MX_E2M3, MX_E3M2 or MX_E2M1
 *   q_data, k_data   packed payload [B, S, H, D*w/8] bytes (w = 8, 6, 6, 4): each
 *               (token, head) row is the little-endian bitstream of its D
 *               elements (mx_quantize_rows' layout with rows = B*S*H, K = D)
 *   q_scale, k_scale ROW32 E8M0 scales [B, S, H, D/32] (the format's scale rule)
 *   other arguments, outputs and errors as mx_attn_fwd; MX_EINVAL also for an
 *   unknown qk_format.  Device pointers 16-byte aligned; async on `stream`.
 */
mx_status mx_attn_fwd_fmt(const uint8_t* q_data, const uint8_t* q_scale,
                          const uint8_t* k_data, const uint8_t* k_scale,
                          const uint8_t* v_data, const uint8_t* v_scale,
                          int B, int S, int H, int D, float softmax_scale, int causal,
                          mx_elem qk_format, void* o, mx_dtype o_dtype, float* lse,
                          hipStream_t stream);

/*
 * mx_attn_fwd_fmt_varlen -- mx_attn_fwd_fmt over packed sequences (the jagged
 * layout of mx_attn_fwd_varlen): Q, K payload rows [T, H, D*w/8] at cu_seqlens
 * token offsets; Q, K ROW32 scale rows [Tp, H, D/32] at the 128-aligned
 * cu_scale_rows offsets (mx_varlen_scale_offsets), pad rows ignored; V as for
 * mx_attn_fwd_varlen; lse [H, T].  Errors as mx_attn_fwd_varlen, and MX_EINVAL
 * for an unknown qk_format.
 */
mx_status mx_attn_fwd_fmt_varlen(const uint8_t* q_data, const uint8_t* q_scale,
                                 const uint8_t* k_data, const uint8_t* k_scale,
                                 const uint8_t* v_data, const uint8_t* v_scale,
                                 const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq,
                                 int total_tokens, int max_seqlen, int H, int D,
                                 float softmax_scale, int causal, mx_elem qk_format,
                                 void* o, mx_dtype o_dtype, float* lse, hipStream_t stream);

/*
 * mx_attn_fwd_bf16 -- BF16 attention forward, the baseline of the pages'
 * speed-up figures ([News], headline comparison with BF16 FlashAttention-4).
 * Reading (the pages do not define it): mx_attn_fwd with every MX step
 * removed; Q, K, V bfloat16; S = Q K^T accumulated in fp32; the same integer
 * frame, p and l as mx_attn_fwd; P rounded to bfloat16 (nearest even) for
 * O = (P V) / l; LSE as mx_attn_fwd.
 *   q, k, v  [B, S, H, D] bfloat16 (device, 16-byte aligned)
 *   D 64 or 128; causal keeps keys j <= i
 *   o        [B, S, H, D], o_dtype MX_BF16 or MX_F32
 *   lse      [B, H, S] fp32, natural log; may be NULL
 * Errors: MX_EINVAL for a bad shape, dtype, scale or alignment; B = 0 or
 * S = 0: MX_OK.  Ownership: all buffers belong to the caller.
 */
mx_status mx_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           int B, int S, int H, int D, float softmax_scale, int causal,
                           void* o, mx_dtype o_dtype, float* lse, hipStream_t stream);

/*
 * mx_attn_fwd_bf16_varlen -- mx_attn_fwd_bf16 over packed sequences
 * ([T, H, D] tensors, cu_seqlens [nseq+1] device int32).  lse is [H, T].
 * max_seqlen bounds every sequence length (host int).
 */
mx_status mx_attn_fwd_bf16_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* cu_seqlens, int nseq, int total_tokens,
                                  int max_seqlen, int H, int D, float softmax_scale, int causal,
                                  void* o, mx_dtype o_dtype, float* lse, hipStream_t stream);

/*
 * mx_attn_bwd_workspace_bytes -- device scratch mx_attn_bwd and
 * mx_attn_bwd_varlen need ([News], forward/backward paragraph: dQ is reduced
 * in FP16 under a static scale, which needs an fp16 accumulator beside the
 * outputs).  Layout (internal): a 256-byte slot holding the fp16 range flag
 * (see mx_attn_bwd_overflow), the fp16 dQ accumulator of tokens x H x D
 * halves (head-major [H, tokens, D]) and D_i [B, H, S] fp32 (or [H, T]), each
 * part 256-byte aligned.  tokens = B*S or T.  Returns 0 for tokens < 0,
 * H < 1 or D < 1.  No allocation; no error state.
 */
size_t mx_attn_bwd_workspace_bytes(int tokens, int H, int D);

/*
 * mx_attn_bwd_overflow -- did the last mx_attn_bwd / mx_attn_bwd_varlen on
 * this workspace leave fp16's range?  The pages keep dQ in FP16 under a
 * static power-of-two scale because dQ values are consistently small ([News],
 * forward/backward paragraph); when they are not, a scaled dQ partial beyond
 * 65504 would saturate and the fp16 accumulator would reach infinity.  The
 * backward detects both on the GPU and records them in the workspace's flag
 * slot (cleared at the start of every backward call with at least one
 * token); the returned dQ is then not valid and the caller should repeat the
 * call with a smaller dq_scale_log2.
 *   workspace  the device workspace the backward was given (16-byte aligned)
 *              (NULL: the calling device's scratch of mx_attn_bwd_noalloc)
 *   overflow   host int: set to 1 if the flag is raised, else 0
 *   stream     the stream the backward ran on: the call copies the flag on it
 *              and synchronizes that stream (it blocks the host).
 * Errors: MX_EINVAL (null or misaligned pointer), MX_EHIP (copy failed).
 */
mx_status mx_attn_bwd_overflow(const void* workspace, int* overflow, hipStream_t stream);

/*
 * mx_attn_bwd_bf16_workspace_bytes -- device scratch mx_attn_bwd_bf16 needs:
 * D_i as fp32 [B, H, S] (or [H, T]), tokens = B*S or T; 256-byte rounded.
 */
size_t mx_attn_bwd_bf16_workspace_bytes(int tokens, int H);

/*
 * mx_attn_bwd_bf16 -- BF16 attention backward, the baseline of the MXFP8
 * backward ([News], headline comparison with BF16 FlashAttention-4).
 * Reading (the pages do not define it): mx_attn_bwd with every MX step
 * removed; p = 2^(S c - fl32(LSE log2 e)) with S = Q K^T in fp32,
 * dP = dO V^T, D_i = sum_d dO_id O_id (fp32), dS = p (dP - D); P and dS
 * rounded to bfloat16 (nearest even) for dV = P^T dO, dK = softmax_scale
 * dS^T Q, dQ = softmax_scale dS K.  dQ is accumulated per query tile (no
 * atomics, deterministic).
 *   q, k, v, o, dout  [B, S, H, D] bfloat16 (o and lse from the forward)
 *   lse               [B, H, S] fp32
 *   dq, dk, dv        [B, S, H, D] in grad_dtype (MX_BF16 or MX_F32)
 *   workspace         >= mx_attn_bwd_bf16_workspace_bytes(B*S, H) bytes
 * Errors: MX_EINVAL (shape, dtype, scale, alignment), MX_EWORKSPACE (missing
 * or short workspace); B = 0 or S = 0: MX_OK.  Ownership: caller's buffers.
 */
mx_status mx_attn_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* o, const uint16_t* dout, const float* lse,
                           int B, int S, int H, int D, float softmax_scale, int causal,
                           void* dq, void* dk, void* dv, mx_dtype grad_dtype,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mx_attn_bwd_bf16_varlen -- mx_attn_bwd_bf16 over packed sequences
 * ([T, H, D] tensors, lse [H, T], cu_seqlens [nseq+1] device int32).
 */
mx_status mx_attn_bwd_bf16_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const uint16_t* o, const uint16_t* dout, const float* lse,
                                  const int32_t* cu_seqlens, int nseq, int total_tokens,
                                  int max_seqlen, int H, int D, float softmax_scale, int causal,
                                  void* dq, void* dk, void* dv, mx_dtype grad_dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mx_attn_bwd -- fused MXFP8 attention backward.
 * Defines: [News], forward/backward paragraph (Q, K, dO quantized in
 * square [32, 32] blocks so one payload feeds both GEMMs; P recomputed;
 * dQ reduced in FP16 under a static scale) and contributions paragraph
 * (dS quantized online in transpose-invariant square blocks); [Blog],
 * "3. Gradient Scale Recomputation in the Backward Pass".
 * Computation per (b, h):
 *   S' = Q^ K^T (SQ32 operands); p = 2^(S' c - fl32(LSE * log2 e));
 *   dP = dO^ V^T (dO^ SQ32, V^ ROW32); D_i = sum_d dO_id O_id (fp32, from
 *   the unquantized dout and o); dS = p (dP - D);
 *   dS^ = MX(dS) in [32 query x 32 key] blocks; P^ = MX(p) in blocks of 32
 *   queries per key;
 *   dV = P^T dO^;  dK = softmax_scale * dS^T Q^;
 *   dQ = softmax_scale * dS^ K^, reduced in fp16 as dQ * 2^dq_scale_log2
 *   and written as acc * 2^-dq_scale_log2.
 *   q_*, k_*, do_*   SQ32 payload + scales; v_* ROW32 payload + scales
 *   o, dout          [B, S, H, D] in io_dtype (MX_BF16 or MX_F32)
 *   lse              [B, H, S] fp32 from the forward
 *   dq_scale_log2    in [-15, 15]
 *   dq, dk, dv       [B, S, H, D] in grad_dtype (MX_BF16 or MX_F32)
 *   workspace        >= mx_attn_bwd_workspace_bytes(B*S, H, D) bytes; a dQ
 *                    partial or accumulator beyond fp16's range raises its
 *                    flag (mx_attn_bwd_overflow), never a status here
 */
mx_status mx_attn_bwd(const uint8_t* q_data, const uint8_t* q_scale,
                      const uint8_t* k_data, const uint8_t* k_scale,
                      const uint8_t* v_data, const uint8_t* v_scale,
                      const uint8_t* do_data, const uint8_t* do_scale,
                      const void* o, const void* dout, mx_dtype io_dtype, const float* lse,
                      int B, int S, int H, int D, float softmax_scale, int causal,
                      int dq_scale_log2,
                      void* dq, void* dk, void* dv, mx_dtype grad_dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mx_attn_bwd_varlen -- mx_attn_bwd over packed sequences.
 * Defines: [News], contributions paragraph (jagged layout: unpadded FP8
 * payload, scales at 128-aligned per-sequence offsets) applied to
 * mx_attn_bwd's computation per sequence.
 *   q_*, k_*, do_*   [T, H, D] payloads, SQ32 scales [Tpad/32, H, D/32]
 *   v_*              [T, H, D] payload, ROW32 scales [Tpad, H, D/32]
 *   o, dout          [T, H, D] in io_dtype; lse [H, T] fp32
 *   cu_seqlens, cu_scale_rows   device int32 [nseq+1]
 *   dq, dk, dv       [T, H, D] in grad_dtype
 *   workspace        >= mx_attn_bwd_workspace_bytes(T, H, D) bytes
 * Causality within each sequence.  Errors: as mx_attn_bwd, and MX_EINVAL for
 * nseq < 1 or null offset arrays; T = 0 or max_seqlen = 0: MX_OK.
 */
mx_status mx_attn_bwd_varlen(const uint8_t* q_data, const uint8_t* q_scale,
                             const uint8_t* k_data, const uint8_t* k_scale,
                             const uint8_t* v_data, const uint8_t* v_scale,
                             const uint8_t* do_data, const uint8_t* do_scale,
                             const void* o, const void* dout, mx_dtype io_dtype, const float* lse,
                             const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq,
                             int total_tokens, int max_seqlen, int H, int D,
                             float softmax_scale, int causal, int dq_scale_log2,
                             void* dq, void* dk, void* dv, mx_dtype grad_dtype,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mx_attn_bwd_fmt -- mx_attn_bwd with Q and K in MXFP6 or MXFP4.
 * Defines: mx_attn_bwd's computation ([News], forward/backward and contributions
 * paragraphs) with the block-scaled MMA's other element formats ([News],
 * paragraph on the block-scaled MMA: MXFP8, MXFP6, MXFP4), read as the OCP MX
 * elements for Q and K only: their square [32, 32] blocks carry E2M3, E3M2 or
 * E2M1 codes (mx_quantize_sq_fmt); dO and V stay MXFP8, and P and dS are
 * quantized online in MXFP8 as in mx_attn_bwd.  Every product takes its
 * operands through the matrix instruction's format fields.
 *   q_row, k_row     [B, S, H, D*w/8] row-packed payloads (mx_quantize_sq_fmt)
 *   q_col, k_col     [B, ceil(S/32), H, D, 32*w/8] column-packed payloads
 *   q_scale, k_scale [B, ceil(S/32), H, D/32] square-block E8M0 scales
 *   qk_format        MX_E2M3, MX_E3M2 or MX_E2M1 (D = 128), or MX_E4M3: then
 *                    exactly mx_attn_bwd with q_row/k_row as the SQ32
 *                    payloads (q_col, k_col unused, may be NULL)
 *   everything else  as mx_attn_bwd
 * Errors: as mx_attn_bwd, and MX_EINVAL for another format, D != 128 with a
 * small format, or a null or misaligned column-packed payload.
 */
mx_status mx_attn_bwd_fmt(const uint8_t* q_row, const uint8_t* q_col, const uint8_t* q_scale,
                          const uint8_t* k_row, const uint8_t* k_col, const uint8_t* k_scale,
                          const uint8_t* v_data, const uint8_t* v_scale,
                          const uint8_t* do_data, const uint8_t* do_scale,
                          const void* o, const void* dout, mx_dtype io_dtype, const float* lse,
                          int B, int S, int H, int D, float softmax_scale, int causal,
                          int dq_scale_log2, mx_elem qk_format,
                          void* dq, void* dk, void* dv, mx_dtype grad_dtype,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mx_attn_bwd_fmt_varlen -- mx_attn_bwd_fmt over packed sequences ([News],
 * contributions paragraph, jagged layout): q_row, k_row [T, H, D*w/8];
 * q_col, k_col [Tpad/32, H, D, 32*w/8] and the scales [Tpad/32, H, D/32] at
 * the 128-aligned per-sequence block rows (mx_quantize_sq_fmt_varlen); the
 * rest as mx_attn_bwd_varlen.  Errors: as mx_attn_bwd_fmt and
 * mx_attn_bwd_varlen.
 */
mx_status mx_attn_bwd_fmt_varlen(const uint8_t* q_row, const uint8_t* q_col, const uint8_t* q_scale,
                                 const uint8_t* k_row, const uint8_t* k_col, const uint8_t* k_scale,
                                 const uint8_t* v_data, const uint8_t* v_scale,
                                 const uint8_t* do_data, const uint8_t* do_scale,
                                 const void* o, const void* dout, mx_dtype io_dtype, const float* lse,
                                 const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq,
                                 int total_tokens, int max_seqlen, int H, int D,
                                 float softmax_scale, int causal, int dq_scale_log2, mx_elem qk_format,
                                 void* dq, void* dk, void* dv, mx_dtype grad_dtype,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * mx_attn_bwd_noalloc -- mx_attn_bwd for callers that cannot allocate device
 * memory or hand in a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, computation and
 * errors as mx_attn_bwd, without the workspace: the range flag, fp16 dQ
 * accumulator and D_i live in a static device array of the library, one per
 * GPU, 128 MiB each (MX_NOALLOC_MAX_BYTES), held until the process ends.
 * Calls whose mx_attn_bwd_workspace_bytes(B*S, H, D) exceeds it return
 * MX_EWORKSPACE before anything is launched (D = 128: up to 516 000 token-head
 * rows, e.g. B4 S4096 H16 or B2 S8192 H16 fit, B4 S8192 H16 does not).  The call allocates nothing and clears what must
 * start at zero with kernels on the stream.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (different streams, threads)
 * race and must be serialized by the caller.  The range flag is read with
 * mx_attn_bwd_overflow(NULL, ...) on the same device.
 */
#define MX_NOALLOC_MAX_BYTES ((size_t)128 << 20)
mx_status mx_attn_bwd_noalloc(const uint8_t* q_data, const uint8_t* q_scale,
                              const uint8_t* k_data, const uint8_t* k_scale,
                              const uint8_t* v_data, const uint8_t* v_scale,
                              const uint8_t* do_data, const uint8_t* do_scale,
                              const void* o, const void* dout, mx_dtype io_dtype, const float* lse,
                              int B, int S, int H, int D, float softmax_scale, int causal,
                              int dq_scale_log2,
                              void* dq, void* dk, void* dv, mx_dtype grad_dtype,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFA_H */
