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

hipError_t launch_quantize(const void* x, bool fp32, int D, const QuantArgs& a, hipStream_t st);
hipError_t launch_scale_offsets(const int32_t* cu, int nseq, int32_t* csr, hipStream_t st);
hipError_t launch_attn_fwd(int D, bool causal, bool out_bf16, FwdArgs a, int max_len, hipStream_t st);

}  // namespace mxk
