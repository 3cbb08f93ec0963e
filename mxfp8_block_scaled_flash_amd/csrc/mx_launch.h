// Kernel argument blocks and launchers (host <-> device boundary inside the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mx_common.h"

namespace mxk {

struct QuantArgs {
  SeqMap seq;
  int H;
  int nseq;
  long nwaves;        // one wave per (sequence or batch, 32-token block, head)
  unsigned layouts;   // bit 0 ROW32, bit 1 COL32, bit 2 SQ32
  uint8_t *row_data, *row_scale, *col_data, *col_scale, *sq_data, *sq_scale;
  const float* gamma; // RMSNorm gain [D] (fused RMSNorm + quantize only)
  double eps;         // RMSNorm epsilon
};

struct FwdArgs {
  const uint8_t *q, *qs, *k, *ks, *v, *vs;
  SeqMap seq;
  int H;
  int nseq;       // batch (fixed) or number of sequences (varlen)
  int nqt;        // query tiles per sequence
  int T;          // total tokens (varlen LSE stride)
  float c;        // fl32(softmax_scale * log2 e)
  void* o;
  float* lse;
};

struct GemmArgs {
  const uint8_t *a, *as, *b, *bs;   // A [M, K], B [N, K] packed payloads; ROW32 scales [M, K/32], [N, K/32]
  int M, N, K;
  int fmt;                          // element format of A and B (matrix-instruction code: 0, 2, 3, 4)
  int tm, tn;                       // tiles along M and N (set by the launcher)
  unsigned layouts;                 // output layouts of C = A B^T
  uint8_t *row_data, *row_scale, *col_data, *col_scale, *sq_data, *sq_scale;
  float* c32;                       // optional fp32 copy of C [M, N]
};

struct BwdArgs {
  const uint8_t *q, *qs, *k, *ks, *v, *vs, *dob, *dos;   // SQ32 Q, K, dO; ROW32 V
  const uint8_t *qc, *kc;   // small-format Q, K: column-packed copies [block row][H][D][32 w / 8]
  const void* o;        // forward output [tokens, H, D]
  const void* dout;     // incoming gradient [tokens, H, D]
  const float* lse;     // [B, H, S] or [H, T]
  SeqMap seq;
  int H;
  int nseq;
  int nkt;              // key tiles per sequence
  int T;                // total tokens
  float c;              // fl32(softmax_scale * log2 e)
  float sigma;          // softmax_scale
  float dq_mult;        // softmax_scale * 2^s
  float dq_unscale;     // 2^-s
  int grad_f32;
  void *dq, *dk, *dv;
  void* acc;            // fp16 dQ accumulator [tokens, H, D] (workspace)
  float* Dbuf;          // D_i (workspace), indexed like lse
  uint32_t* ovf;        // fp16 dQ range flag (workspace): set to 1 when a scaled partial or the
                        // accumulator leaves fp16's finite range (MX path only)
};

hipError_t launch_quantize(const void* x, bool fp32, int D, bool rmsnorm, const QuantArgs& a, hipStream_t st);
hipError_t launch_scale_offsets(const int32_t* cu, int nseq, int32_t* csr, hipStream_t st);
hipError_t launch_attn_fwd(int D, bool causal, bool out_bf16, int qk_fmt, FwdArgs a, int max_len, hipStream_t st);
hipError_t launch_attn_fwd_bf16(int D, bool causal, bool out_bf16, FwdArgs a, int max_len, hipStream_t st);
hipError_t launch_attn_bwd(int D, bool causal, bool io_f32, BwdArgs a, int max_len, hipStream_t st, int qk_fmt = 0);
hipError_t launch_bwd_pre(int D, bool io_f32, const BwdArgs& a, hipStream_t st);
hipError_t launch_attn_bwd_bf16(int D, bool causal, BwdArgs a, int max_len, hipStream_t st);
hipError_t launch_quantize_rows(const void* x, bool fp32, long rows, int K, int fmt, uint8_t* data, uint8_t* scale,
                                hipStream_t st);
hipError_t launch_quantize_rows_varlen(const void* x, bool fp32, const int32_t* cu, const int32_t* csr, int nseq,
                                       long total_scale_rows, int H, int K, int fmt, uint8_t* data, uint8_t* scale,
                                       hipStream_t st);
hipError_t launch_gemm_quantize(GemmArgs a, hipStream_t st);
hipError_t launch_quantize_sq_fmt(const void* x, bool fp32, const int32_t* cu, const int32_t* csr, int nseq, int S,
                                  long nrows, int H, int D, int fmt, uint8_t* row_data, uint8_t* col_data,
                                  uint8_t* scale, hipStream_t st);

}  // namespace mxk
