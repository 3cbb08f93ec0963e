// Host side of the C ABI declared in include/mxfa.h: argument validation,
// launch geometry and status codes.  Nothing here allocates device memory or
// synchronises the host; every kernel goes onto the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/mxfa.h"
#include "mx_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// gfx950 check, cached per device ordinal (0 unknown, 1 gfx950, 2 other).
std::atomic<int> g_dev_ok[64];

mx_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MX_EHIP;
  if (dev < 0 || dev >= 64) return MX_EUNSUPPORTED;
  int st = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MX_EHIP;
    st = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_ok[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? MX_OK : MX_EUNSUPPORTED;
}

mx_status from_hip(hipError_t e) { return e == hipSuccess ? MX_OK : MX_EHIP; }

bool valid_layouts(unsigned layouts) { return layouts != 0 && (layouts & ~7u) == 0; }

bool layout_ptrs_ok(unsigned layouts, uint8_t* rd, uint8_t* rs, uint8_t* cd, uint8_t* cs, uint8_t* sd,
                    uint8_t* ss) {
  if ((layouts & MX_ROW32) && !(rd && rs && aligned16(rd) && aligned16(rs))) return false;
  if ((layouts & MX_COL32) && !(cd && cs && aligned16(cd) && aligned16(cs))) return false;
  if ((layouts & MX_SQ32) && !(sd && ss && aligned16(sd) && aligned16(ss))) return false;
  return true;
}

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p || !aligned16(p)) return false;
  return true;
}

float log2_scale(float softmax_scale) { return softmax_scale * 1.44269504088896340736f; }

constexpr long kMaxElems = 1L << 40;
// Token indices and per-tile byte spans are 32-bit inside the kernels: at most 2^31 - 1 tokens
// per call, and at most 2^16 heads (so a 128-row tile of one head spans less than 2^31 bytes).
constexpr long kMaxTokens = (1L << 31) - 1;
constexpr int kMaxHeads = 1 << 16;

}  // namespace

extern "C" {

int mx_abi_version(void) { return MXFA_ABI_VERSION; }

const char* mx_status_str(mx_status s) {
  switch (s) {
    case MX_OK: return "MX_OK";
    case MX_EINVAL: return "MX_EINVAL: invalid argument";
    case MX_EUNSUPPORTED: return "MX_EUNSUPPORTED: unsupported device or combination";
    case MX_EHIP: return "MX_EHIP: HIP runtime error";
    case MX_EWORKSPACE: return "MX_EWORKSPACE: workspace missing or too small";
  }
  return "unknown mx_status";
}

}  // extern "C"

namespace {

// Shared by the plain and the fused RMSNorm quantizers (gamma == nullptr: plain).
mx_status quantize_fixed(const void* x, mx_dtype x_dtype, const float* gamma, float eps, int B, int S, int H, int D,
                         unsigned layouts, uint8_t* row32_data, uint8_t* row32_scale, uint8_t* col32_data,
                         uint8_t* col32_scale, uint8_t* sq32_data, uint8_t* sq32_scale, hipStream_t stream) {
  if (B < 0 || S < 0 || H < 1 || H > kMaxHeads || (D != 64 && D != 128)) return MX_EINVAL;
  if (x_dtype != MX_BF16 && x_dtype != MX_F32) return MX_EINVAL;
  if (!valid_layouts(layouts)) return MX_EINVAL;
  if ((long)B * S * H * D > kMaxElems || (long)B * S > kMaxTokens) return MX_EINVAL;
  if ((long)B * S == 0) return MX_OK;
  if (!x || !aligned16(x)) return MX_EINVAL;
  if (!layout_ptrs_ok(layouts, row32_data, row32_scale, col32_data, col32_scale, sq32_data, sq32_scale))
    return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  mxk::QuantArgs a{};
  a.seq.cu = nullptr;
  a.seq.csr = nullptr;
  a.seq.S = S;
  a.seq.nblk = (S + 31) / 32;
  a.H = H;
  a.nseq = B;
  a.nwaves = (long)B * a.seq.nblk * H;
  a.layouts = layouts;
  a.row_data = row32_data; a.row_scale = row32_scale;
  a.col_data = col32_data; a.col_scale = col32_scale;
  a.sq_data = sq32_data; a.sq_scale = sq32_scale;
  a.gamma = gamma;
  a.eps = (double)eps;
  return from_hip(mxk::launch_quantize(x, x_dtype == MX_F32, D, gamma != nullptr, a, stream));
}

mx_status quantize_jagged(const void* x, mx_dtype x_dtype, const float* gamma, float eps, const int32_t* cu_seqlens,
                          const int32_t* cu_scale_rows, int nseq, int total_tokens, int total_scale_rows, int H, int D,
                          unsigned layouts, uint8_t* row32_data, uint8_t* row32_scale, uint8_t* col32_data,
                          uint8_t* col32_scale, uint8_t* sq32_data, uint8_t* sq32_scale, hipStream_t stream) {
  if (nseq < 1 || total_tokens < 0 || total_scale_rows < 0 || total_scale_rows % 128 != 0) return MX_EINVAL;
  if (total_scale_rows < total_tokens) return MX_EINVAL;
  if (H < 1 || H > kMaxHeads || (D != 64 && D != 128)) return MX_EINVAL;
  if (x_dtype != MX_BF16 && x_dtype != MX_F32) return MX_EINVAL;
  if (!valid_layouts(layouts)) return MX_EINVAL;
  if (!cu_seqlens || !cu_scale_rows) return MX_EINVAL;
  if ((long)total_scale_rows * H * D > kMaxElems) return MX_EINVAL;
  if (total_scale_rows == 0) return MX_OK;
  if (total_tokens > 0 && (!x || !aligned16(x))) return MX_EINVAL;
  if (!layout_ptrs_ok(layouts, row32_data, row32_scale, col32_data, col32_scale, sq32_data, sq32_scale))
    return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  mxk::QuantArgs a{};
  a.seq.cu = cu_seqlens;
  a.seq.csr = cu_scale_rows;
  a.seq.S = 0;
  a.seq.nblk = 0;
  a.H = H;
  a.nseq = nseq;
  a.nwaves = (long)(total_scale_rows / 32) * H;
  a.layouts = layouts;
  a.row_data = row32_data; a.row_scale = row32_scale;
  a.col_data = col32_data; a.col_scale = col32_scale;
  a.sq_data = sq32_data; a.sq_scale = sq32_scale;
  a.gamma = gamma;
  a.eps = (double)eps;
  return from_hip(mxk::launch_quantize(x, x_dtype == MX_F32, D, gamma != nullptr, a, stream));
}

bool valid_norm(const float* gamma, float eps) {
  return gamma && (reinterpret_cast<uintptr_t>(gamma) & 3u) == 0 && std::isfinite(eps) && eps >= 0.f;
}

}  // namespace

extern "C" {

mx_status mx_quantize(const void* x, mx_dtype x_dtype, int B, int S, int H, int D, unsigned layouts,
                      uint8_t* row32_data, uint8_t* row32_scale, uint8_t* col32_data, uint8_t* col32_scale,
                      uint8_t* sq32_data, uint8_t* sq32_scale, hipStream_t stream) {
  return quantize_fixed(x, x_dtype, nullptr, 0.f, B, S, H, D, layouts, row32_data, row32_scale, col32_data,
                        col32_scale, sq32_data, sq32_scale, stream);
}

mx_status mx_rmsnorm_quantize(const void* x, mx_dtype x_dtype, const float* gamma, float eps, int B, int S, int H,
                              int D, unsigned layouts, uint8_t* row32_data, uint8_t* row32_scale,
                              uint8_t* col32_data, uint8_t* col32_scale, uint8_t* sq32_data, uint8_t* sq32_scale,
                              hipStream_t stream) {
  if (!valid_norm(gamma, eps)) return MX_EINVAL;
  return quantize_fixed(x, x_dtype, gamma, eps, B, S, H, D, layouts, row32_data, row32_scale, col32_data,
                        col32_scale, sq32_data, sq32_scale, stream);
}

mx_status mx_varlen_scale_offsets(const int32_t* cu_seqlens, int nseq, int32_t* cu_scale_rows, hipStream_t stream) {
  if (nseq < 1 || !cu_seqlens || !cu_scale_rows) return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  return from_hip(mxk::launch_scale_offsets(cu_seqlens, nseq, cu_scale_rows, stream));
}

mx_status mx_quantize_varlen(const void* x, mx_dtype x_dtype, const int32_t* cu_seqlens, const int32_t* cu_scale_rows,
                             int nseq, int total_tokens, int total_scale_rows, int H, int D, unsigned layouts,
                             uint8_t* row32_data, uint8_t* row32_scale, uint8_t* col32_data, uint8_t* col32_scale,
                             uint8_t* sq32_data, uint8_t* sq32_scale, hipStream_t stream) {
  return quantize_jagged(x, x_dtype, nullptr, 0.f, cu_seqlens, cu_scale_rows, nseq, total_tokens, total_scale_rows,
                         H, D, layouts, row32_data, row32_scale, col32_data, col32_scale, sq32_data, sq32_scale,
                         stream);
}

mx_status mx_rmsnorm_quantize_varlen(const void* x, mx_dtype x_dtype, const float* gamma, float eps,
                                     const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq,
                                     int total_tokens, int total_scale_rows, int H, int D, unsigned layouts,
                                     uint8_t* row32_data, uint8_t* row32_scale, uint8_t* col32_data,
                                     uint8_t* col32_scale, uint8_t* sq32_data, uint8_t* sq32_scale,
                                     hipStream_t stream) {
  if (!valid_norm(gamma, eps)) return MX_EINVAL;
  return quantize_jagged(x, x_dtype, gamma, eps, cu_seqlens, cu_scale_rows, nseq, total_tokens, total_scale_rows,
                         H, D, layouts, row32_data, row32_scale, col32_data, col32_scale, sq32_data, sq32_scale,
                         stream);
}

static bool valid_elem(int f) { return f == MX_E4M3 || f == MX_E2M3 || f == MX_E3M2 || f == MX_E2M1; }

mx_status mx_quantize_rows(const void* x, mx_dtype x_dtype, int rows, int K, mx_elem format, uint8_t* data,
                           uint8_t* scale, hipStream_t stream) {
  if (rows < 0 || K < 32 || K % 32 != 0 || !valid_elem(format)) return MX_EINVAL;
  if (x_dtype != MX_BF16 && x_dtype != MX_F32) return MX_EINVAL;
  if ((long)rows * K > kMaxElems) return MX_EINVAL;
  if (rows == 0) return MX_OK;
  if (!all_aligned({x, data}) || !scale) return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  return from_hip(mxk::launch_quantize_rows(x, x_dtype == MX_F32, rows, K, (int)format, data, scale, stream));
}

mx_status mx_quantize_rows_varlen(const void* x, mx_dtype x_dtype, const int32_t* cu_seqlens,
                                  const int32_t* cu_scale_rows, int nseq, int total_tokens, int total_scale_rows,
                                  int H, int K, mx_elem format, uint8_t* data, uint8_t* scale, hipStream_t stream) {
  if (nseq < 1 || total_tokens < 0 || total_scale_rows < 0 || !cu_seqlens || !cu_scale_rows) return MX_EINVAL;
  if (H < 1 || H > kMaxHeads || K < 32 || K % 32 != 0 || !valid_elem(format)) return MX_EINVAL;
  if (x_dtype != MX_BF16 && x_dtype != MX_F32) return MX_EINVAL;
  if ((long)total_scale_rows * H * K > kMaxElems || (long)total_tokens * H * K > kMaxElems) return MX_EINVAL;
  if (total_scale_rows < total_tokens || total_scale_rows % 128 != 0) return MX_EINVAL;
  if (total_tokens == 0) return MX_OK;
  if (!all_aligned({x, data}) || !scale) return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  return from_hip(mxk::launch_quantize_rows_varlen(x, x_dtype == MX_F32, cu_seqlens, cu_scale_rows, nseq,
                                                   total_scale_rows, H, K, (int)format, data, scale, stream));
}

static bool small_elem(int f) { return f == MX_E2M3 || f == MX_E3M2 || f == MX_E2M1; }

mx_status mx_quantize_sq_fmt(const void* x, mx_dtype x_dtype, int B, int S, int H, int D, mx_elem format,
                             uint8_t* row_data, uint8_t* col_data, uint8_t* scale, hipStream_t stream) {
  if (B < 0 || S < 0 || H < 1 || H > kMaxHeads || (D != 64 && D != 128) || !small_elem(format)) return MX_EINVAL;
  if (x_dtype != MX_BF16 && x_dtype != MX_F32) return MX_EINVAL;
  const long nrows = (long)B * ((S + 31) / 32);
  if ((long)B * S * H * D > kMaxElems || nrows * 32 * H * D > kMaxElems || nrows * H > 2147483647L) return MX_EINVAL;
  if ((long)B * S == 0) return MX_OK;
  if (!all_aligned({x, row_data, col_data}) || !scale) return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  return from_hip(mxk::launch_quantize_sq_fmt(x, x_dtype == MX_F32, nullptr, nullptr, B, S, nrows, H, D, (int)format,
                                              row_data, col_data, scale, stream));
}

mx_status mx_quantize_sq_fmt_varlen(const void* x, mx_dtype x_dtype, const int32_t* cu_seqlens,
                                    const int32_t* cu_scale_rows, int nseq, int total_tokens, int total_scale_rows,
                                    int H, int D, mx_elem format, uint8_t* row_data, uint8_t* col_data,
                                    uint8_t* scale, hipStream_t stream) {
  if (nseq < 1 || total_tokens < 0 || total_scale_rows < 0 || !cu_seqlens || !cu_scale_rows) return MX_EINVAL;
  if (H < 1 || H > kMaxHeads || (D != 64 && D != 128) || !small_elem(format)) return MX_EINVAL;
  if (x_dtype != MX_BF16 && x_dtype != MX_F32) return MX_EINVAL;
  if ((long)total_scale_rows * H * D > kMaxElems || (long)total_tokens * H * D > kMaxElems) return MX_EINVAL;
  if (total_scale_rows < total_tokens || total_scale_rows % 128 != 0) return MX_EINVAL;
  if ((long)(total_scale_rows / 32) * H > 2147483647L) return MX_EINVAL;
  if (total_tokens == 0) return MX_OK;
  if (!all_aligned({x, row_data, col_data}) || !scale) return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  return from_hip(mxk::launch_quantize_sq_fmt(x, x_dtype == MX_F32, cu_seqlens, cu_scale_rows, nseq, 0,
                                              (long)total_scale_rows / 32, H, D, (int)format, row_data, col_data,
                                              scale, stream));
}

mx_status mx_gemm_quantize(const uint8_t* a_data, const uint8_t* a_scale, const uint8_t* b_data,
                           const uint8_t* b_scale, mx_elem ab_format, int M, int N, int K, unsigned layouts,
                           uint8_t* c_row32_data,
                           uint8_t* c_row32_scale, uint8_t* c_col32_data, uint8_t* c_col32_scale,
                           uint8_t* c_sq32_data, uint8_t* c_sq32_scale, float* c_f32, hipStream_t stream) {
  // K bounded so that a 128-row tile of an operand stays within 32-bit buffer offsets
  if (M < 0 || N < 0 || K < 64 || K > (1 << 20) || K % 64 != 0 || N % 16 != 0) return MX_EINVAL;
  if ((layouts & ~7u) != 0 || (layouts == 0 && !c_f32)) return MX_EINVAL;
  if (!valid_elem(ab_format)) return MX_EINVAL;
  if ((long)M * K > kMaxElems || (long)N * K > kMaxElems || (long)M * N > kMaxElems) return MX_EINVAL;
  if ((long)M * N == 0) return MX_OK;
  if (!all_aligned({a_data, a_scale, b_data, b_scale})) return MX_EINVAL;
  if (layouts && !layout_ptrs_ok(layouts, c_row32_data, c_row32_scale, c_col32_data, c_col32_scale, c_sq32_data,
                                 c_sq32_scale))
    return MX_EINVAL;
  if (c_f32 && !aligned16(c_f32)) return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  mxk::GemmArgs a{};
  a.a = a_data; a.as = a_scale; a.b = b_data; a.bs = b_scale;
  a.M = M; a.N = N; a.K = K;
  a.fmt = (int)ab_format;
  a.layouts = layouts;
  a.row_data = c_row32_data; a.row_scale = c_row32_scale;
  a.col_data = c_col32_data; a.col_scale = c_col32_scale;
  a.sq_data = c_sq32_data; a.sq_scale = c_sq32_scale;
  a.c32 = c_f32;
  return from_hip(mxk::launch_gemm_quantize(a, stream));
}

static mx_status fwd_common(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data,
                            const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale, int H, int D,
                            float softmax_scale, void* o, mx_dtype o_dtype, mxk::FwdArgs& a) {
  if (H < 1 || H > kMaxHeads || (D != 64 && D != 128)) return MX_EINVAL;
  if (o_dtype != MX_BF16 && o_dtype != MX_F32) return MX_EINVAL;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MX_EINVAL;
  if (!all_aligned({q_data, q_scale, k_data, k_scale, v_data, v_scale, o})) return MX_EINVAL;
  a.q = q_data; a.qs = q_scale; a.k = k_data; a.ks = k_scale; a.v = v_data; a.vs = v_scale;
  a.H = H;
  a.c = log2_scale(softmax_scale);
  a.o = o;
  return MX_OK;
}

static mx_status attn_fwd_fixed(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data,
                                const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale, int B, int S,
                                int H, int D, float softmax_scale, int causal, int qk_fmt, void* o,
                                mx_dtype o_dtype, float* lse, hipStream_t stream) {
  if (!valid_elem(qk_fmt)) return MX_EINVAL;
  if (B < 0 || S < 0) return MX_EINVAL;
  if ((long)B * S * H * D > kMaxElems || (long)B * S > kMaxTokens) return MX_EINVAL;
  if ((long)B * S == 0) return MX_OK;
  mxk::FwdArgs a{};
  if (mx_status st = fwd_common(q_data, q_scale, k_data, k_scale, v_data, v_scale, H, D, softmax_scale, o, o_dtype, a))
    return st;
  if (lse && !aligned16(lse)) return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  a.seq.cu = nullptr;
  a.seq.csr = nullptr;
  a.seq.S = S;
  a.seq.nblk = (S + 31) / 32;
  a.nseq = B;
  a.T = B * S;
  a.lse = lse;
  return from_hip(mxk::launch_attn_fwd(D, causal != 0, o_dtype == MX_BF16, qk_fmt, a, S, stream));
}

mx_status mx_attn_fwd(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data, const uint8_t* k_scale,
                      const uint8_t* v_data, const uint8_t* v_scale, int B, int S, int H, int D,
                      float softmax_scale, int causal, void* o, mx_dtype o_dtype, float* lse, hipStream_t stream) {
  return attn_fwd_fixed(q_data, q_scale, k_data, k_scale, v_data, v_scale, B, S, H, D, softmax_scale, causal, MX_E4M3,
                        o, o_dtype, lse, stream);
}

mx_status mx_attn_fwd_fmt(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data,
                          const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale, int B, int S, int H,
                          int D, float softmax_scale, int causal, mx_elem qk_format, void* o, mx_dtype o_dtype,
                          float* lse, hipStream_t stream) {
  return attn_fwd_fixed(q_data, q_scale, k_data, k_scale, v_data, v_scale, B, S, H, D, softmax_scale, causal,
                        (int)qk_format, o, o_dtype, lse, stream);
}

static mx_status attn_fwd_jagged(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data,
                                 const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale,
                                 const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq, int total_tokens,
                                 int max_seqlen, int H, int D, float softmax_scale, int causal, int qk_fmt, void* o,
                                 mx_dtype o_dtype, float* lse, hipStream_t stream) {
  if (!valid_elem(qk_fmt)) return MX_EINVAL;
  if (nseq < 1 || total_tokens < 0 || max_seqlen < 0 || !cu_seqlens || !cu_scale_rows) return MX_EINVAL;
  if ((long)total_tokens * H * D > kMaxElems) return MX_EINVAL;
  if (total_tokens == 0 || max_seqlen == 0) return MX_OK;
  mxk::FwdArgs a{};
  if (mx_status st = fwd_common(q_data, q_scale, k_data, k_scale, v_data, v_scale, H, D, softmax_scale, o, o_dtype, a))
    return st;
  if (lse && !aligned16(lse)) return MX_EINVAL;
  if (mx_status st = check_device()) return st;
  a.seq.cu = cu_seqlens;
  a.seq.csr = cu_scale_rows;
  a.seq.S = 0;
  a.seq.nblk = 0;
  a.nseq = nseq;
  a.T = total_tokens;
  a.lse = lse;
  return from_hip(mxk::launch_attn_fwd(D, causal != 0, o_dtype == MX_BF16, qk_fmt, a, max_seqlen, stream));
}

mx_status mx_attn_fwd_varlen(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data,
                             const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale,
                             const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq, int total_tokens,
                             int max_seqlen, int H, int D, float softmax_scale, int causal, void* o,
                             mx_dtype o_dtype, float* lse, hipStream_t stream) {
  return attn_fwd_jagged(q_data, q_scale, k_data, k_scale, v_data, v_scale, cu_seqlens, cu_scale_rows, nseq,
                         total_tokens, max_seqlen, H, D, softmax_scale, causal, MX_E4M3, o, o_dtype, lse, stream);
}

mx_status mx_attn_fwd_fmt_varlen(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data,
                                 const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale,
                                 const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq, int total_tokens,
                                 int max_seqlen, int H, int D, float softmax_scale, int causal, mx_elem qk_format,
                                 void* o, mx_dtype o_dtype, float* lse, hipStream_t stream) {
  return attn_fwd_jagged(q_data, q_scale, k_data, k_scale, v_data, v_scale, cu_seqlens, cu_scale_rows, nseq,
                         total_tokens, max_seqlen, H, D, softmax_scale, causal, (int)qk_format, o, o_dtype, lse,
                         stream);
}

static mx_status fwd_bf16_common(const uint16_t* q, const uint16_t* k, const uint16_t* v, int H, int D,
                                 float softmax_scale, void* o, mx_dtype o_dtype, float* lse, mxk::FwdArgs& a) {
  if (H < 1 || H > kMaxHeads || (D != 64 && D != 128)) return MX_EINVAL;
  if (o_dtype != MX_BF16 && o_dtype != MX_F32) return MX_EINVAL;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MX_EINVAL;
  if (!all_aligned({q, k, v, o})) return MX_EINVAL;
  if (lse && !aligned16(lse)) return MX_EINVAL;
  a.q = (const uint8_t*)q; a.k = (const uint8_t*)k; a.v = (const uint8_t*)v;
  a.H = H;
  a.c = log2_scale(softmax_scale);
  a.o = o;
  a.lse = lse;
  return MX_OK;
}

mx_status mx_attn_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int S, int H, int D,
                           float softmax_scale, int causal, void* o, mx_dtype o_dtype, float* lse,
                           hipStream_t stream) {
  if (B < 0 || S < 0) return MX_EINVAL;
  if ((long)B * S * H * D > kMaxElems || (long)B * S > kMaxTokens) return MX_EINVAL;
  if ((long)B * S == 0) return MX_OK;
  mxk::FwdArgs a{};
  if (mx_status st = fwd_bf16_common(q, k, v, H, D, softmax_scale, o, o_dtype, lse, a)) return st;
  if (mx_status st = check_device()) return st;
  a.seq.S = S;
  a.seq.nblk = (S + 31) / 32;
  a.nseq = B;
  a.T = B * S;
  return from_hip(mxk::launch_attn_fwd_bf16(D, causal != 0, o_dtype == MX_BF16, a, S, stream));
}

mx_status mx_attn_fwd_bf16_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                  const int32_t* cu_seqlens, int nseq, int total_tokens, int max_seqlen, int H,
                                  int D, float softmax_scale, int causal, void* o, mx_dtype o_dtype, float* lse,
                                  hipStream_t stream) {
  if (nseq < 1 || total_tokens < 0 || max_seqlen < 0 || !cu_seqlens) return MX_EINVAL;
  if ((long)total_tokens * H * D > kMaxElems) return MX_EINVAL;
  if (total_tokens == 0 || max_seqlen == 0) return MX_OK;
  mxk::FwdArgs a{};
  if (mx_status st = fwd_bf16_common(q, k, v, H, D, softmax_scale, o, o_dtype, lse, a)) return st;
  if (mx_status st = check_device()) return st;
  a.seq.cu = cu_seqlens;
  a.seq.csr = cu_seqlens;   // no scale rows in this path; the map only needs a readable array
  a.nseq = nseq;
  a.T = total_tokens;
  return from_hip(mxk::launch_attn_fwd_bf16(D, causal != 0, o_dtype == MX_BF16, a, max_seqlen, stream));
}

// Backward workspace: the fp16 range flag (one 256-byte slot at offset 0), the fp16 dQ accumulator,
// D_i; each part 256-byte aligned.
static constexpr size_t kFlagBytes = 256;

size_t mx_attn_bwd_workspace_bytes(int tokens, int H, int D) {
  if (tokens < 0 || H < 1 || D < 1) return 0;
  auto up = [](size_t v) { return (v + 255) / 256 * 256; };
  return kFlagBytes + up((size_t)tokens * H * D * 2) + up((size_t)tokens * H * 4);
}

static mx_status scratch_ptr(void** out);

mx_status mx_attn_bwd_overflow(const void* workspace, int* overflow, hipStream_t stream) {
  if (!overflow || (workspace && !aligned16(workspace))) return MX_EINVAL;
  if (!workspace) {   // the calling device's scratch (mx_attn_bwd_noalloc)
    void* p = nullptr;
    if (mx_status st = scratch_ptr(&p)) return st;
    workspace = p;
  }
  uint32_t flag = 0;
  if (hipMemcpyAsync(&flag, workspace, sizeof(flag), hipMemcpyDeviceToHost, stream) != hipSuccess) return MX_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return MX_EHIP;
  *overflow = flag != 0;
  return MX_OK;
}

static mx_status bwd_common(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data,
                            const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale,
                            const uint8_t* do_data, const uint8_t* do_scale, const void* o, const void* dout,
                            mx_dtype io_dtype, const float* lse, int H, int D, float softmax_scale, int dq_scale_log2,
                            void* dq, void* dk, void* dv, mx_dtype grad_dtype, void* workspace,
                            size_t workspace_bytes, int tokens, mxk::BwdArgs& a) {
  if (H < 1 || H > kMaxHeads || (D != 64 && D != 128)) return MX_EINVAL;
  if ((io_dtype != MX_BF16 && io_dtype != MX_F32) || (grad_dtype != MX_BF16 && grad_dtype != MX_F32)) return MX_EINVAL;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MX_EINVAL;
  if (dq_scale_log2 < -15 || dq_scale_log2 > 15) return MX_EINVAL;
  if (!all_aligned({q_data, q_scale, k_data, k_scale, v_data, v_scale, do_data, do_scale, o, dout, lse, dq, dk, dv}))
    return MX_EINVAL;
  if (!workspace || !aligned16(workspace)) return MX_EWORKSPACE;
  if (workspace_bytes < mx_attn_bwd_workspace_bytes(tokens, H, D)) return MX_EWORKSPACE;
  a.q = q_data; a.qs = q_scale; a.k = k_data; a.ks = k_scale; a.v = v_data; a.vs = v_scale;
  a.dob = do_data; a.dos = do_scale;
  a.o = o; a.dout = dout; a.lse = lse;
  a.H = H;
  a.c = log2_scale(softmax_scale);
  a.sigma = softmax_scale;
  a.dq_mult = softmax_scale * std::ldexp(1.0f, dq_scale_log2);
  a.dq_unscale = std::ldexp(1.0f, -dq_scale_log2);
  a.grad_f32 = grad_dtype == MX_F32;
  a.dq = dq; a.dk = dk; a.dv = dv;
  const size_t acc_bytes = ((size_t)tokens * H * D * 2 + 255) / 256 * 256;
  a.ovf = static_cast<uint32_t*>(workspace);
  a.acc = static_cast<uint8_t*>(workspace) + kFlagBytes;
  a.Dbuf = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + kFlagBytes + acc_bytes);
  return MX_OK;
}

size_t mx_attn_bwd_bf16_workspace_bytes(int tokens, int H) {
  if (tokens < 0 || H < 1) return 0;
  return ((size_t)tokens * H * 4 + 255) / 256 * 256;
}

static mx_status bwd_bf16_common(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                                 const uint16_t* dout, const float* lse, int H, int D, float softmax_scale, void* dq,
                                 void* dk, void* dv, mx_dtype grad_dtype, void* workspace, size_t workspace_bytes,
                                 int tokens, mxk::BwdArgs& a) {
  if (H < 1 || H > kMaxHeads || (D != 64 && D != 128)) return MX_EINVAL;
  if (grad_dtype != MX_BF16 && grad_dtype != MX_F32) return MX_EINVAL;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MX_EINVAL;
  if (!all_aligned({q, k, v, o, dout, lse, dq, dk, dv})) return MX_EINVAL;
  if (!workspace || !aligned16(workspace)) return MX_EWORKSPACE;
  if (workspace_bytes < mx_attn_bwd_bf16_workspace_bytes(tokens, H)) return MX_EWORKSPACE;
  a.q = (const uint8_t*)q; a.k = (const uint8_t*)k; a.v = (const uint8_t*)v;
  a.o = o; a.dout = dout; a.lse = lse;
  a.H = H;
  a.c = log2_scale(softmax_scale);
  a.sigma = softmax_scale;
  a.grad_f32 = grad_dtype == MX_F32;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.acc = nullptr;
  a.Dbuf = static_cast<float*>(workspace);
  return MX_OK;
}

mx_status mx_attn_bwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                           const uint16_t* dout, const float* lse, int B, int S, int H, int D, float softmax_scale,
                           int causal, void* dq, void* dk, void* dv, mx_dtype grad_dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || S < 0) return MX_EINVAL;
  if ((long)B * S * H * D > kMaxElems || (long)B * S > kMaxTokens) return MX_EINVAL;
  if ((long)B * S == 0) return MX_OK;
  mxk::BwdArgs a{};
  if (mx_status st = bwd_bf16_common(q, k, v, o, dout, lse, H, D, softmax_scale, dq, dk, dv, grad_dtype, workspace,
                                     workspace_bytes, B * S, a))
    return st;
  if (mx_status st = check_device()) return st;
  a.seq.S = S;
  a.seq.nblk = (S + 31) / 32;
  a.nseq = B;
  a.T = B * S;
  return from_hip(mxk::launch_attn_bwd_bf16(D, causal != 0, a, S, stream));
}

mx_status mx_attn_bwd_bf16_varlen(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                                  const uint16_t* dout, const float* lse, const int32_t* cu_seqlens, int nseq,
                                  int total_tokens, int max_seqlen, int H, int D, float softmax_scale, int causal,
                                  void* dq, void* dk, void* dv, mx_dtype grad_dtype, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  if (nseq < 1 || total_tokens < 0 || max_seqlen < 0 || !cu_seqlens) return MX_EINVAL;
  if ((long)total_tokens * H * D > kMaxElems) return MX_EINVAL;
  if (total_tokens == 0 || max_seqlen == 0) return MX_OK;
  mxk::BwdArgs a{};
  if (mx_status st = bwd_bf16_common(q, k, v, o, dout, lse, H, D, softmax_scale, dq, dk, dv, grad_dtype, workspace,
                                     workspace_bytes, total_tokens, a))
    return st;
  if (mx_status st = check_device()) return st;
  a.seq.cu = cu_seqlens;
  a.seq.csr = cu_seqlens;   // no scale rows in this path
  a.nseq = nseq;
  a.T = total_tokens;
  return from_hip(mxk::launch_attn_bwd_bf16(D, causal != 0, a, max_seqlen, stream));
}

mx_status mx_attn_bwd(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data, const uint8_t* k_scale,
                      const uint8_t* v_data, const uint8_t* v_scale, const uint8_t* do_data, const uint8_t* do_scale,
                      const void* o, const void* dout, mx_dtype io_dtype, const float* lse, int B, int S, int H, int D,
                      float softmax_scale, int causal, int dq_scale_log2, void* dq, void* dk, void* dv,
                      mx_dtype grad_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (B < 0 || S < 0) return MX_EINVAL;
  if ((long)B * S * H * D > kMaxElems || (long)B * S > kMaxTokens) return MX_EINVAL;
  if ((long)B * S == 0) return MX_OK;
  mxk::BwdArgs a{};
  if (mx_status st = bwd_common(q_data, q_scale, k_data, k_scale, v_data, v_scale, do_data, do_scale, o, dout,
                                io_dtype, lse, H, D, softmax_scale, dq_scale_log2, dq, dk, dv, grad_dtype, workspace,
                                workspace_bytes, B * S, a))
    return st;
  if (mx_status st = check_device()) return st;
  a.seq.cu = nullptr;
  a.seq.csr = nullptr;
  a.seq.S = S;
  a.seq.nblk = (S + 31) / 32;
  a.nseq = B;
  a.T = B * S;
  return from_hip(mxk::launch_attn_bwd(D, causal != 0, io_dtype == MX_F32, a, S, stream));
}

mx_status mx_attn_bwd_varlen(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data,
                             const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale,
                             const uint8_t* do_data, const uint8_t* do_scale, const void* o, const void* dout,
                             mx_dtype io_dtype, const float* lse, const int32_t* cu_seqlens,
                             const int32_t* cu_scale_rows, int nseq, int total_tokens, int max_seqlen, int H, int D,
                             float softmax_scale, int causal, int dq_scale_log2, void* dq, void* dk, void* dv,
                             mx_dtype grad_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (nseq < 1 || total_tokens < 0 || max_seqlen < 0 || !cu_seqlens || !cu_scale_rows) return MX_EINVAL;
  if ((long)total_tokens * H * D > kMaxElems) return MX_EINVAL;
  if (total_tokens == 0 || max_seqlen == 0) return MX_OK;
  mxk::BwdArgs a{};
  if (mx_status st = bwd_common(q_data, q_scale, k_data, k_scale, v_data, v_scale, do_data, do_scale, o, dout,
                                io_dtype, lse, H, D, softmax_scale, dq_scale_log2, dq, dk, dv, grad_dtype, workspace,
                                workspace_bytes, total_tokens, a))
    return st;
  if (mx_status st = check_device()) return st;
  a.seq.cu = cu_seqlens;
  a.seq.csr = cu_scale_rows;
  a.seq.S = 0;
  a.seq.nblk = 0;
  a.nseq = nseq;
  a.T = total_tokens;
  return from_hip(mxk::launch_attn_bwd(D, causal != 0, io_dtype == MX_F32, a, max_seqlen, stream));
}

mx_status mx_attn_bwd_fmt(const uint8_t* q_row, const uint8_t* q_col, const uint8_t* q_scale, const uint8_t* k_row,
                          const uint8_t* k_col, const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale,
                          const uint8_t* do_data, const uint8_t* do_scale, const void* o, const void* dout,
                          mx_dtype io_dtype, const float* lse, int B, int S, int H, int D, float softmax_scale,
                          int causal, int dq_scale_log2, mx_elem qk_format, void* dq, void* dk, void* dv,
                          mx_dtype grad_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (qk_format == MX_E4M3)
    return mx_attn_bwd(q_row, q_scale, k_row, k_scale, v_data, v_scale, do_data, do_scale, o, dout, io_dtype, lse, B,
                       S, H, D, softmax_scale, causal, dq_scale_log2, dq, dk, dv, grad_dtype, workspace,
                       workspace_bytes, stream);
  if (!small_elem(qk_format) || D != 128) return MX_EINVAL;
  if (B < 0 || S < 0) return MX_EINVAL;
  if ((long)B * S * H * D > kMaxElems || (long)B * S > kMaxTokens) return MX_EINVAL;
  if ((long)B * S == 0) return MX_OK;
  if (!all_aligned({q_col, k_col})) return MX_EINVAL;
  mxk::BwdArgs a{};
  if (mx_status st = bwd_common(q_row, q_scale, k_row, k_scale, v_data, v_scale, do_data, do_scale, o, dout,
                                io_dtype, lse, H, D, softmax_scale, dq_scale_log2, dq, dk, dv, grad_dtype, workspace,
                                workspace_bytes, B * S, a))
    return st;
  if (mx_status st = check_device()) return st;
  a.qc = q_col;
  a.kc = k_col;
  a.seq.cu = nullptr;
  a.seq.csr = nullptr;
  a.seq.S = S;
  a.seq.nblk = (S + 31) / 32;
  a.nseq = B;
  a.T = B * S;
  return from_hip(mxk::launch_attn_bwd(D, causal != 0, io_dtype == MX_F32, a, S, stream, (int)qk_format));
}

mx_status mx_attn_bwd_fmt_varlen(const uint8_t* q_row, const uint8_t* q_col, const uint8_t* q_scale,
                                 const uint8_t* k_row, const uint8_t* k_col, const uint8_t* k_scale,
                                 const uint8_t* v_data, const uint8_t* v_scale, const uint8_t* do_data,
                                 const uint8_t* do_scale, const void* o, const void* dout, mx_dtype io_dtype,
                                 const float* lse, const int32_t* cu_seqlens, const int32_t* cu_scale_rows, int nseq,
                                 int total_tokens, int max_seqlen, int H, int D, float softmax_scale, int causal,
                                 int dq_scale_log2, mx_elem qk_format, void* dq, void* dk, void* dv,
                                 mx_dtype grad_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (qk_format == MX_E4M3)
    return mx_attn_bwd_varlen(q_row, q_scale, k_row, k_scale, v_data, v_scale, do_data, do_scale, o, dout, io_dtype,
                              lse, cu_seqlens, cu_scale_rows, nseq, total_tokens, max_seqlen, H, D, softmax_scale,
                              causal, dq_scale_log2, dq, dk, dv, grad_dtype, workspace, workspace_bytes, stream);
  if (!small_elem(qk_format) || D != 128) return MX_EINVAL;
  if (nseq < 1 || total_tokens < 0 || max_seqlen < 0 || !cu_seqlens || !cu_scale_rows) return MX_EINVAL;
  if ((long)total_tokens * H * D > kMaxElems) return MX_EINVAL;
  if (total_tokens == 0 || max_seqlen == 0) return MX_OK;
  if (!all_aligned({q_col, k_col})) return MX_EINVAL;
  mxk::BwdArgs a{};
  if (mx_status st = bwd_common(q_row, q_scale, k_row, k_scale, v_data, v_scale, do_data, do_scale, o, dout,
                                io_dtype, lse, H, D, softmax_scale, dq_scale_log2, dq, dk, dv, grad_dtype, workspace,
                                workspace_bytes, total_tokens, a))
    return st;
  if (mx_status st = check_device()) return st;
  a.qc = q_col;
  a.kc = k_col;
  a.seq.cu = cu_seqlens;
  a.seq.csr = cu_scale_rows;
  a.seq.S = 0;
  a.seq.nblk = 0;
  a.nseq = nseq;
  a.T = total_tokens;
  return from_hip(mxk::launch_attn_bwd(D, causal != 0, io_dtype == MX_F32, a, max_seqlen, stream, (int)qk_format));
}

// ---------------------------------------------------------------- no-allocation backward
// The backward's scratch (range flag, fp16 dQ accumulator, D_i) for callers that cannot allocate:
// one file-scope device array, so each GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not device memory: its device
// address comes from hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to a kernel or a copy.
static constexpr size_t kScratchBytes = MX_NOALLOC_MAX_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[64];   // device address of `scratch`, per device ordinal

static mx_status scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MX_EHIP;
  if (dev < 0 || dev >= 64) return MX_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MX_EHIP;
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MX_OK;
}

mx_status mx_attn_bwd_noalloc(const uint8_t* q_data, const uint8_t* q_scale, const uint8_t* k_data,
                              const uint8_t* k_scale, const uint8_t* v_data, const uint8_t* v_scale,
                              const uint8_t* do_data, const uint8_t* do_scale, const void* o, const void* dout,
                              mx_dtype io_dtype, const float* lse, int B, int S, int H, int D,
                              float softmax_scale, int causal, int dq_scale_log2, void* dq, void* dk, void* dv,
                              mx_dtype grad_dtype, hipStream_t stream) {
  if (B < 0 || S < 0) return MX_EINVAL;
  if ((long)B * S * H * D > kMaxElems || (long)B * S > kMaxTokens) return MX_EINVAL;
  if ((long)B * S == 0) return MX_OK;
  const size_t need = mx_attn_bwd_workspace_bytes(B * S, H, D);
  // the arguments are checked (against an aligned stand-in workspace) before the device is touched
  mxk::BwdArgs a{};
  if (mx_status st = bwd_common(q_data, q_scale, k_data, k_scale, v_data, v_scale, do_data, do_scale, o, dout,
                                io_dtype, lse, H, D, softmax_scale, dq_scale_log2, dq, dk, dv, grad_dtype,
                                reinterpret_cast<void*>(static_cast<uintptr_t>(256)), need, B * S, a))
    return st;
  if (need > kScratchBytes) return MX_EWORKSPACE;
  if (mx_status st = check_device()) return st;
  void* ws = nullptr;
  if (mx_status st = scratch_ptr(&ws)) return st;
  return mx_attn_bwd(q_data, q_scale, k_data, k_scale, v_data, v_scale, do_data, do_scale, o, dout, io_dtype, lse,
                     B, S, H, D, softmax_scale, causal, dq_scale_log2, dq, dk, dv, grad_dtype, ws, need, stream);
}

}  // extern "C"
