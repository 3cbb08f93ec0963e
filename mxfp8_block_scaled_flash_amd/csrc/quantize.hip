// One-pass MX quantization: ROW32, COL32 and SQ32 payloads and scales from a
// single read of a bf16 or fp32 activation tile.
//
// The block format is the pages' MXFP8 ("Low-Precision FlashAttention-4 ...
// for NVIDIA Blackwell", section "Understanding OCP MXFP8 Microscaling on
// Blackwell"): 32 elements, one E8M0 scale, E4M3 payload.  Emitting several
// scale layouts in one pass is the producer design of "Low Precision Flash
// Attention 4: End-to-End Block-Scaled Attention for Blackwell",
// contributions paragraph; the jagged variant keeps the payload at packed
// token positions and pads only the scale rows to 128-row boundaries (same
// paragraph).
//
// The fused RMSNorm + quantize variant (the same paragraph's "fused RMSNorm +
// Quantize" producer) normalizes each (token, head) row over D first:
// rstd = fl32(1 / sqrt(sum(x^2) / D + eps)) with the sum of squares, the
// division, the square root and the reciprocal in fp64 (the squares of bf16 or
// fp32 inputs are exact there), then y = fl32(fl32(x rstd) gamma), and
// quantizes y.
//
// Work unit: one wavefront per (sequence, 32-token block, head): a 32 x D
// tile, read once with 16-byte loads (row = D contiguous elements), reduced
// for all three block shapes in registers (cross-lane steps by shuffles), and
// written once per requested layout.  The kernel is HBM-bound; encoding uses
// an exact power-of-two ldexp, a clamp to +-448 (the hardware convert does
// not saturate) and the hardware round-to-nearest-even fp8 convert.
#include "mx_common.h"
#include "mx_launch.h"

namespace mxk {

template <typename T, int D, bool NORM>
__global__ __launch_bounds__(256) void quantize_kernel(const T* __restrict__ x, QuantArgs a) {
  constexpr int ES = sizeof(T);
  constexpr int CPR = D * ES / 16;   // 16-byte chunks per token row
  constexpr int EPC = 16 / ES;       // elements per chunk
  constexpr int RPP = 64 / CPR;      // token rows per wave-wide load
  constexpr int NP = kBlock / RPP;   // loads per lane
  constexpr int LPB = kBlock / EPC;  // lanes per 32-feature block
  constexpr int NDB = D / kBlock;    // feature blocks per row
  const int lane = threadIdx.x & 63;
  const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave >= a.nwaves) return;
  const int h = (int)(wave % a.H);
  const long g = wave / a.H;

  int s, blk;
  if (a.seq.cu) {  // padded block index -> sequence by binary search of the scale offsets
    const long row = g * kBlock;
    int lo = 0, hi = a.nseq;  // find the last s with csr[s] <= row
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
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
  const bool varlen = a.seq.cu != nullptr;

  const int cc = lane % CPR;   // chunk within the row
  const int r0 = lane / CPR;   // first row of this lane

  float v[NP][EPC];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int t = blk * kBlock + r0 + RPP * p;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (t < L) w = *reinterpret_cast<const uint4*>(x + ((long)(tok0 + t) * a.H + h) * D + cc * EPC);
    if constexpr (ES == 2) {
      v[p][0] = bf16_lo(w.x); v[p][1] = bf16_hi(w.x);
      v[p][2] = bf16_lo(w.y); v[p][3] = bf16_hi(w.y);
      v[p][4] = bf16_lo(w.z); v[p][5] = bf16_hi(w.z);
      v[p][6] = bf16_lo(w.w); v[p][7] = bf16_hi(w.w);
    } else {
      v[p][0] = __uint_as_float(w.x); v[p][1] = __uint_as_float(w.y);
      v[p][2] = __uint_as_float(w.z); v[p][3] = __uint_as_float(w.w);
    }
  }

  if constexpr (NORM) {
    // ---- RMSNorm of each row over D: the row's CPR lanes are neighbours
    float gm[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) gm[e] = a.gamma[cc * EPC + e];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      double ss = 0.0;
#pragma unroll
      for (int e = 0; e < EPC; ++e) ss += (double)v[p][e] * (double)v[p][e];
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
      const float rstd = (float)(1.0 / sqrt(ss / (double)D + a.eps));
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[p][e] = (v[p][e] * rstd) * gm[e];
    }
  }

  // ---- block maxima
  float rmax[NP];  // per row, over this lane's 32-feature block
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) m = fmaxf(m, fabsf(v[p][e]));
#pragma unroll
    for (int o = 1; o < LPB; o <<= 1) m = wave_max_xor(m, o);
    rmax[p] = m;
  }
  float cmax[EPC];  // per feature, over the 32 rows
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    float m = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) m = fmaxf(m, fabsf(v[p][e]));
#pragma unroll
    for (int o = CPR; o < 64; o <<= 1) m = wave_max_xor(m, o);
    cmax[e] = m;
  }
  float smax = 0.f;  // per 32 x 32 square
#pragma unroll
  for (int p = 0; p < NP; ++p) smax = fmaxf(smax, rmax[p]);
#pragma unroll
  for (int o = CPR; o < 64; o <<= 1) smax = wave_max_xor(smax, o);

  auto enc4 = [](const float* y, int sh0, int sh1, int sh2, int sh3) -> uint32_t {
    // y * 2^sh, clamp to +-448, RNE convert; four codes packed little-endian
    float a0 = __builtin_amdgcn_fmed3f(ldexpf(y[0], sh0), -448.f, 448.f);
    float a1 = __builtin_amdgcn_fmed3f(ldexpf(y[1], sh1), -448.f, 448.f);
    float a2 = __builtin_amdgcn_fmed3f(ldexpf(y[2], sh2), -448.f, 448.f);
    float a3 = __builtin_amdgcn_fmed3f(ldexpf(y[3], sh3), -448.f, 448.f);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, r, true);
    return (uint32_t)r;
  };

  const long pay_row = (long)a.H * D;
  // ---- ROW32
  if (a.layouts & 1) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int t = blk * kBlock + r0 + RPP * p;
      const int k = scale_code(rmax[p]);
      const int sh = 127 - k;
      if (t < L) {
        uint8_t* dst = a.row_data + (long)(tok0 + t) * pay_row + (long)h * D + cc * EPC;
        if constexpr (EPC == 8) {
          uint2 o2 = make_uint2(enc4(&v[p][0], sh, sh, sh, sh), enc4(&v[p][4], sh, sh, sh, sh));
          *reinterpret_cast<uint2*>(dst) = o2;
        } else {
          *reinterpret_cast<uint32_t*>(dst) = enc4(&v[p][0], sh, sh, sh, sh);
        }
      }
      if (cc % LPB == 0 && (t < L || varlen)) {
        long row = varlen ? (long)srow0 + t : (long)tok0 + t;
        a.row_scale[(row * a.H + h) * NDB + cc / LPB] = (uint8_t)(t < L ? k : 0);
      }
    }
  }
  // ---- COL32
  if (a.layouts & 2) {
    int sh[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) sh[e] = 127 - scale_code(cmax[e]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int t = blk * kBlock + r0 + RPP * p;
      if (t < L) {
        uint8_t* dst = a.col_data + (long)(tok0 + t) * pay_row + (long)h * D + cc * EPC;
        if constexpr (EPC == 8) {
          uint2 o2 = make_uint2(enc4(&v[p][0], sh[0], sh[1], sh[2], sh[3]),
                                enc4(&v[p][4], sh[4], sh[5], sh[6], sh[7]));
          *reinterpret_cast<uint2*>(dst) = o2;
        } else {
          *reinterpret_cast<uint32_t*>(dst) = enc4(&v[p][0], sh[0], sh[1], sh[2], sh[3]);
        }
      }
    }
    if (r0 == 0) {
      uint8_t* dst = a.col_scale + ((long)(sblk0 + blk) * a.H + h) * D + cc * EPC;
#pragma unroll
      for (int e = 0; e < EPC; ++e) dst[e] = (uint8_t)(127 - sh[e]);
    }
  }
  // ---- SQ32
  if (a.layouts & 4) {
    const int k = scale_code(smax);
    const int sh = 127 - k;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int t = blk * kBlock + r0 + RPP * p;
      if (t < L) {
        uint8_t* dst = a.sq_data + (long)(tok0 + t) * pay_row + (long)h * D + cc * EPC;
        if constexpr (EPC == 8) {
          uint2 o2 = make_uint2(enc4(&v[p][0], sh, sh, sh, sh), enc4(&v[p][4], sh, sh, sh, sh));
          *reinterpret_cast<uint2*>(dst) = o2;
        } else {
          *reinterpret_cast<uint32_t*>(dst) = enc4(&v[p][0], sh, sh, sh, sh);
        }
      }
    }
    if (r0 == 0 && cc % LPB == 0)
      a.sq_scale[((long)(sblk0 + blk) * a.H + h) * NDB + cc / LPB] = (uint8_t)k;
  }
}

__global__ void scale_offsets_kernel(const int32_t* __restrict__ cu, int nseq, int32_t* __restrict__ csr) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    int32_t acc = 0;
    csr[0] = 0;
    for (int s = 0; s < nseq; ++s) {
      int32_t L = cu[s + 1] - cu[s];
      acc += (L + 127) / 128 * 128;
      csr[s + 1] = acc;
    }
  }
}

template <bool NORM>
static void launch_quantize_t(const void* x, bool fp32, int D, const QuantArgs& a, dim3 grid, dim3 block,
                              hipStream_t st) {
  if (fp32) {
    if (D == 64) quantize_kernel<float, 64, NORM><<<grid, block, 0, st>>>((const float*)x, a);
    else quantize_kernel<float, 128, NORM><<<grid, block, 0, st>>>((const float*)x, a);
  } else {
    if (D == 64) quantize_kernel<uint16_t, 64, NORM><<<grid, block, 0, st>>>((const uint16_t*)x, a);
    else quantize_kernel<uint16_t, 128, NORM><<<grid, block, 0, st>>>((const uint16_t*)x, a);
  }
}

hipError_t launch_quantize(const void* x, bool fp32, int D, bool rmsnorm, const QuantArgs& a, hipStream_t st) {
  if (a.nwaves == 0) return hipSuccess;
  dim3 grid((unsigned)((a.nwaves + 3) / 4)), block(256);
  if (rmsnorm) launch_quantize_t<true>(x, fp32, D, a, grid, block, st);
  else launch_quantize_t<false>(x, fp32, D, a, grid, block, st);
  return hipGetLastError();
}

hipError_t launch_scale_offsets(const int32_t* cu, int nseq, int32_t* csr, hipStream_t st) {
  scale_offsets_kernel<<<1, 64, 0, st>>>(cu, nseq, csr);
  return hipGetLastError();
}

}  // namespace mxk
