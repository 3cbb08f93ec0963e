// MX quantization of GEMM operands in any element format of the block-scaled
// matrix instruction: MXFP8 (E4M3), MXFP6 (E2M3, E3M2) and MXFP4 (E2M1),
// blocks of 32 along each row (the contraction axis), payload packed as the
// instruction reads it.  The pages name these formats beside MXFP8 ("Low
// Precision Flash Attention 4: End-to-End Block-Scaled Attention for
// Blackwell", paragraph on the block-scaled MMA instructions); the element
// definitions are the OCP MX ones.
//
// One thread per 32-element block: the block's 64 (bf16) or 128 (fp32) bytes
// are contiguous and neighbouring threads read neighbouring blocks.  The
// scale is read off amax's exponent field; elements are scaled by an exact
// power of two and encoded with integer arithmetic (round to nearest even,
// saturating), so every code is the exactly rounded one.  Packing: element j
// of a row at bits [w j, w j + w) of a little-endian bitstream (w = 8, 6, 4).
#include "mx_common.h"
#include "mx_launch.h"

namespace mxk {

namespace {

// format: exponent bits, mantissa bits, bias, emax (exponent of the largest power of two), largest code
template <int FMT>
struct Fmt;
template <>
struct Fmt<0> { static constexpr int EB = 4, MB = 3, BIAS = 7, EMAX = 8, W = 8; static constexpr uint32_t TOP = 0x7E; static constexpr float MAXV = 448.f; };
template <>
struct Fmt<2> { static constexpr int EB = 2, MB = 3, BIAS = 1, EMAX = 2, W = 6; static constexpr uint32_t TOP = 0x1F; static constexpr float MAXV = 7.5f; };
template <>
struct Fmt<3> { static constexpr int EB = 3, MB = 2, BIAS = 3, EMAX = 4, W = 6; static constexpr uint32_t TOP = 0x1F; static constexpr float MAXV = 28.f; };
template <>
struct Fmt<4> { static constexpr int EB = 2, MB = 1, BIAS = 1, EMAX = 2, W = 4; static constexpr uint32_t TOP = 0x7; static constexpr float MAXV = 6.f; };

// y already scaled into the format's range (exactly); returns the element code
template <int FMT>
MX_DEV uint32_t encode(float y) {
  using F = Fmt<FMT>;
  const float a = fabsf(y);
  const uint32_t sign = (__float_as_uint(y) >> 31) << (F::EB + F::MB);
  // binade of a, floored at the subnormal binade (fp32 zero/subnormal inputs give -127: floored too)
  int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;
  e = max(e, 1 - F::BIAS);
  float r = rintf(ldexpf(a, F::MB - e));   // a / spacing, round to nearest even (exact scaling)
  if (r >= (float)(2 << F::MB)) {          // carry into the next binade
    e += 1;
    r = (float)(1 << F::MB);
  }
  const int ri = (int)r;
  const bool sub = ri < (1 << F::MB);
  const uint32_t E = sub ? 0u : (uint32_t)(e + F::BIAS);
  const uint32_t M = sub ? (uint32_t)ri : (uint32_t)(ri - (1 << F::MB));
  uint32_t code = (E << F::MB) | M;
  if (a > F::MAXV || E > (uint32_t)((1 << F::EB) - 1)) code = F::TOP;
  return code | sign;
}

// One 32-element block: src (32 elements) -> W dwords of packed codes at dst, E8M0 scale at *sc.
template <typename T, int FMT>
MX_DEV void quantize_block(const T* __restrict__ src, uint8_t* __restrict__ dst_bytes, uint8_t* __restrict__ sc) {
  using F = Fmt<FMT>;
  float v[32];
  if constexpr (sizeof(T) == 2) {
    const uint4* p = (const uint4*)src;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 u = p[c];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * c + 2 * i] = bf16_lo(w4[i]);
        v[8 * c + 2 * i + 1] = bf16_hi(w4[i]);
      }
    }
  } else {
    const float4* p = (const float4*)src;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float4 f = p[c];
      v[4 * c] = f.x; v[4 * c + 1] = f.y; v[4 * c + 2] = f.z; v[4 * c + 3] = f.w;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  // E8M0 = clamp(floor(log2 amax) - EMAX + 127, 0, 254); zero and fp32-subnormal amax give 0
  const int ea = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  const int k = ea == 0 ? 0 : min(max(ea - F::EMAX, 0), 254);
  const int sh = 127 - k;
  uint32_t out[F::W] = {};   // 32 codes x W bits = W dwords
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = encode<FMT>(ldexpf(v[i], sh));
    const int pos = F::W * i, wd = pos >> 5, bit = pos & 31;
    out[wd] |= c << bit;
    if (bit + F::W > 32) out[wd + 1] |= c >> (32 - bit);
  }
  uint32_t* dst = (uint32_t*)dst_bytes;
  if constexpr (F::W == 8) {
    ((uint4*)dst)[0] = make_uint4(out[0], out[1], out[2], out[3]);
    ((uint4*)dst)[1] = make_uint4(out[4], out[5], out[6], out[7]);
  } else if constexpr (F::W == 6) {
    ((uint2*)dst)[0] = make_uint2(out[0], out[1]);
    ((uint2*)dst)[1] = make_uint2(out[2], out[3]);
    ((uint2*)dst)[2] = make_uint2(out[4], out[5]);
  } else {
    ((uint4*)dst)[0] = make_uint4(out[0], out[1], out[2], out[3]);
  }
  *sc = (uint8_t)k;
}

template <typename T, int FMT>
__global__ __launch_bounds__(256) void quantize_rows_kernel(const T* __restrict__ x, long nblk, uint8_t* __restrict__ data,
                                                            uint8_t* __restrict__ scale) {
  const long b = (long)blockIdx.x * 256 + threadIdx.x;   // block index = row * (K/32) + block in row
  if (b >= nblk) return;
  quantize_block<T, FMT>(x + b * 32, data + b * (4 * Fmt<FMT>::W), scale + b);
}

// Jagged rows: one thread per (scale row, head, 32-element block) of the padded scale tensor
// [Tp, H, K/32].  Scale row r belongs to the sequence s with cu_scale_rows[s] <= r <
// cu_scale_rows[s+1] (binary search; empty sequences own no row); a row past the sequence's length
// is padding and gets scale 0, a row inside it quantizes token cu_seqlens[s] + (r - cu_scale_rows[s]),
// whose payload stays at its packed position.
template <typename T, int FMT>
__global__ __launch_bounds__(256) void quantize_rows_varlen_kernel(const T* __restrict__ x, const int32_t* __restrict__ cu,
                                                                   const int32_t* __restrict__ csr, int nseq, int H,
                                                                   int kb, long nblk, uint8_t* __restrict__ data,
                                                                   uint8_t* __restrict__ scale) {
  const long b = (long)blockIdx.x * 256 + threadIdx.x;   // ((r * H) + h) * kb + j
  if (b >= nblk) return;
  const long rh = b / kb;
  const int j = (int)(b - rh * kb);
  const int r = (int)(rh / H), h = (int)(rh - (long)r * H);
  int lo = 0, hi = nseq - 1;   // largest s in [0, nseq) with csr[s] <= r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (csr[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int t_in = r - csr[lo];
  if (t_in >= cu[lo + 1] - cu[lo]) {
    scale[b] = 0;
    return;
  }
  const long src = ((long)(cu[lo] + t_in) * H + h) * kb + j;   // block index in the packed payload
  quantize_block<T, FMT>(x + src * 32, data + src * (4 * Fmt<FMT>::W), scale + b);
}


// Square [32 tokens x 32 features] blocks in a small element format (E2M3, E3M2, E2M1): the backward's
// Q and K operands with MXFP6 / MXFP4 payloads (its square blocks: "Low Precision Flash Attention 4",
// forward/backward paragraph; the formats: the same page's paragraph on the block-scaled MMA).  A
// packed payload cannot be read across its rows the way a byte payload can, so each block is written
// twice: row-packed (token rows along D, as mx_quantize_rows) and column-packed (for each feature, the
// block's 32 tokens as one packed 32-element block), both from the same codes and one E8M0 scale.
// One wave per block: lane l holds token row l / 2, features 16 (l % 2) .. +15; the column copy goes
// through a 1 KB LDS transpose per wave.
struct SqFmtArgs {
  SeqMap seq;
  int H, nseq;
  long nrows;                     // padded 32-token block rows (fixed: B ceil(S/32); jagged: Tpad / 32)
  uint8_t *row_data, *col_data, *scale;
};

template <int W>
MX_DEV void pack16(const uint32_t (&c)[16], uint32_t (&o)[W / 2]) {
#pragma unroll
  for (int j = 0; j < W / 2; ++j) o[j] = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int pos = W * i, wd = pos >> 5, bit = pos & 31;
    o[wd] |= c[i] << bit;
    if (bit + W > 32) o[wd + 1] |= c[i] >> (32 - bit);
  }
}

template <typename T, int FMT, int D>
__global__ __launch_bounds__(64 * D / 32) void quantize_sq_fmt_kernel(const T* __restrict__ x, SqFmtArgs a) {
  using F = Fmt<FMT>;
  constexpr int W = F::W, BB = 32 * W / 8, HB = BB / 2, KRB = D * W / 8;
  __shared__ __attribute__((aligned(16))) uint8_t tc[D / 32][32][32];   // per wave: codes [feature][token]
  const int lane = threadIdx.x & 63, fb = threadIdx.x >> 6;
  const int h = (int)(blockIdx.x % a.H);
  const long g = blockIdx.x / a.H;         // padded block row
  int s, blk;
  if (a.seq.cu) {  // padded block row -> sequence: the last s with csr[s] <= 32 g
    const long row = g * 32;
    int lo = 0, hi = a.nseq;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((long)a.seq.csr[mid] <= row) lo = mid; else hi = mid;
    }
    s = lo;
    blk = (int)(g - (a.seq.csr[s] >> 5));
  } else {
    s = (int)(g / a.seq.nblk);
    blk = (int)(g % a.seq.nblk);
  }
  int tok0, L, srow0, sblk0;
  a.seq.get(s, tok0, L, srow0, sblk0);
  const int r = lane >> 1, hf = lane & 1;
  const int t = blk * 32 + r;
  float v[16];
  if (t < L) {
    const T* src = x + ((long)(tok0 + t) * a.H + h) * D + fb * 32 + hf * 16;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const uint4 u = ((const uint4*)src)[c];
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          v[8 * c + 2 * i] = bf16_lo(w4[i]);
          v[8 * c + 2 * i + 1] = bf16_hi(w4[i]);
        }
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float4 f = ((const float4*)src)[c];
        v[4 * c] = f.x; v[4 * c + 1] = f.y; v[4 * c + 2] = f.z; v[4 * c + 3] = f.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = wave_max_nonneg(amax);
  // E8M0 = clamp(floor(log2 amax) - EMAX + 127, 0, 254); zero and fp32-subnormal amax give 0
  const int ea = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  const int k = ea == 0 ? 0 : min(max(ea - F::EMAX, 0), 254);
  uint32_t c[16], o[W / 2];
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = encode<FMT>(ldexpf(v[i], 127 - k));
  pack16<W>(c, o);
  if (t < L) {
    uint32_t* dst = (uint32_t*)(a.row_data + ((long)(tok0 + t) * a.H + h) * KRB + fb * BB + hf * HB);
#pragma unroll
    for (int j = 0; j < W / 2; ++j) dst[j] = o[j];
  }
  // column copy: token-major codes of each feature through LDS
#pragma unroll
  for (int i = 0; i < 16; ++i) tc[fb][hf * 16 + i][r] = (uint8_t)c[i];
  __syncthreads();
  const int col = lane >> 1;
  const uint4 u = *(const uint4*)&tc[fb][col][hf * 16];
  const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = (w4[i >> 2] >> (8 * (i & 3))) & 0xFFu;
  pack16<W>(c, o);
  uint32_t* cdst = (uint32_t*)(a.col_data + (((long)(sblk0 + blk) * a.H + h) * D + fb * 32 + col) * BB + hf * HB);
#pragma unroll
  for (int j = 0; j < W / 2; ++j) cdst[j] = o[j];
  if (lane == 0) a.scale[((long)(sblk0 + blk) * a.H + h) * (D / 32) + fb] = (uint8_t)k;
}

}  // namespace

hipError_t launch_quantize_rows(const void* x, bool fp32, long rows, int K, int fmt, uint8_t* data, uint8_t* scale,
                                hipStream_t st) {
  const long nblk = rows * (K / 32);
  if (nblk == 0) return hipSuccess;
  dim3 g((unsigned)((nblk + 255) / 256)), b(256);
#define MX_QR_CASE(F)                                                                                     \
  if (fmt == F) {                                                                                         \
    if (fp32) quantize_rows_kernel<float, F><<<g, b, 0, st>>>((const float*)x, nblk, data, scale);        \
    else quantize_rows_kernel<uint16_t, F><<<g, b, 0, st>>>((const uint16_t*)x, nblk, data, scale);       \
    return hipGetLastError();                                                                             \
  }
  MX_QR_CASE(0) MX_QR_CASE(2) MX_QR_CASE(3) MX_QR_CASE(4)
#undef MX_QR_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_quantize_rows_varlen(const void* x, bool fp32, const int32_t* cu, const int32_t* csr, int nseq,
                                       long total_scale_rows, int H, int K, int fmt, uint8_t* data, uint8_t* scale,
                                       hipStream_t st) {
  const int kb = K / 32;
  const long nblk = total_scale_rows * H * kb;
  if (nblk == 0) return hipSuccess;
  dim3 g((unsigned)((nblk + 255) / 256)), b(256);
#define MX_QRV_CASE(F)                                                                                        \
  if (fmt == F) {                                                                                             \
    if (fp32)                                                                                                 \
      quantize_rows_varlen_kernel<float, F><<<g, b, 0, st>>>((const float*)x, cu, csr, nseq, H, kb, nblk, data, scale); \
    else                                                                                                      \
      quantize_rows_varlen_kernel<uint16_t, F><<<g, b, 0, st>>>((const uint16_t*)x, cu, csr, nseq, H, kb, nblk, data, \
                                                                  scale);                                     \
    return hipGetLastError();                                                                                 \
  }
  MX_QRV_CASE(0) MX_QRV_CASE(2) MX_QRV_CASE(3) MX_QRV_CASE(4)
#undef MX_QRV_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_quantize_sq_fmt(const void* x, bool fp32, const int32_t* cu, const int32_t* csr, int nseq, int S,
                                  long nrows, int H, int D, int fmt, uint8_t* row_data, uint8_t* col_data,
                                  uint8_t* scale, hipStream_t st) {
  SqFmtArgs a{};
  a.seq.cu = cu;
  a.seq.csr = csr;
  a.seq.S = S;
  a.seq.nblk = (S + 31) / 32;
  a.H = H;
  a.nseq = nseq;
  a.nrows = nrows;
  a.row_data = row_data;
  a.col_data = col_data;
  a.scale = scale;
  const long nwg = nrows * H;
  if (nwg == 0) return hipSuccess;
  dim3 g((unsigned)nwg), b((unsigned)(64 * D / 32));
#define MX_QSQ_CASE(F, DD)                                                                              \
  if (fmt == F && D == DD) {                                                                            \
    if (fp32) quantize_sq_fmt_kernel<float, F, DD><<<g, b, 0, st>>>((const float*)x, a);                \
    else quantize_sq_fmt_kernel<uint16_t, F, DD><<<g, b, 0, st>>>((const uint16_t*)x, a);               \
    return hipGetLastError();                                                                           \
  }
  MX_QSQ_CASE(2, 128) MX_QSQ_CASE(3, 128) MX_QSQ_CASE(4, 128) MX_QSQ_CASE(2, 64) MX_QSQ_CASE(3, 64)
  MX_QSQ_CASE(4, 64)
#undef MX_QSQ_CASE
  return hipErrorInvalidValue;
}

}  // namespace mxk
