// BF16 attention forward for gfx950: the baseline the MXFP8 path is measured
// against ("Low Precision Flash Attention 4: End-to-End Block-Scaled Attention
// for Blackwell", headline speed-ups over BF16 FlashAttention-4).
//
// Same computation as the MXFP8 forward with every MX step removed: S = Q K^T
// from bf16 operands in fp32, the log2-domain softmax under a lazily moved
// integer frame (exact power-of-two rescaling of O and l), P rounded to bf16
// (nearest even) for O += P V, l summing the fp32 p.
//
// gfx950 mapping, kept from the MXFP8 kernel so the two differ only in the
// arithmetic:
//  * wave = 32 queries; S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (8 per
//    32-key block at D = 128), so a lane holds one query and 16 keys of each
//    32-key block; the row maximum is in-lane plus one lane-half exchange;
//  * P's bf16 pairs are regrouped between lane halves with v_permlane32_swap
//    so each lane holds 8 consecutive keys per 16-key step, the layout of the
//    instruction's second operand;
//  * V^T comes from the row-major V tile through ds_read_b64_tr_b16: in each
//    16-lane group, lane i receives element i%4 of the 8-byte rows addressed
//    by lanes i/4, i/4+4, i/4+8, i/4+12, so lanes addressing (key row
//    k0 + 4r + L/4, features d0 + 4(L%4)) give lane i feature d0 + i at four
//    consecutive keys;
//  * 64-key K and V tiles double-buffered in LDS (K rows padded by 16 bytes,
//    V rows by 64 so the transpose reads of a half wave touch distinct
//    banks), the next tile's loads in flight during the current one, one
//    barrier per tile, two workgroups per CU, XCD-aware (sequence, head)
//    order, longest causal query tiles first.
#include "mx_common.h"
#include "mx_launch.h"

namespace mxk {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));

MX_DEV v16f mfma_bf16(const v8bf& a, const v8bf& b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

MX_DEV v8bf as_v8bf(uint4 u) { return __builtin_bit_cast(v8bf, u); }

// two fp32 -> bf16 (round to nearest even) in one word, a in the low half
MX_DEV uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

MX_DEV uint2 lds_tr16(const uint8_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)(p)));
}

template <int D>
struct KVStage16 {
  static constexpr int CH = 64 * 2 * D / 16 / 256;   // 16-byte chunks per thread per tensor
  uint4 k[CH], v[CH];
};

}  // namespace

template <int D, bool CAUSAL, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int NW = 4;
  constexpr int BM = 32 * NW;   // queries per workgroup
  constexpr int BN = 64;        // keys per tile
  constexpr int NK = D / 16;    // 16-feature steps of the Q K^T contraction
  constexpr int ND = D / 32;    // 32-feature chunks of O
  constexpr int RB = 2 * D;     // bytes per token row of one head
  constexpr int KSK = RB + 16;  // LDS row stride of K
  constexpr int KSV = RB + 64;  // LDS row stride of V
  constexpr float kLazy = 8.f;
  constexpr int NT = NW * 64;
  constexpr int CPR = RB / 16;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][BN * KSK];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][BN * KSV];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
  const int u = (j / a.nqt) * 8 + xcd;
  if (u >= a.nseq * a.H) return;
  const int qt = a.nqt - 1 - (j % a.nqt);
  const int h = __builtin_amdgcn_readfirstlane(u % a.H), s = __builtin_amdgcn_readfirstlane(u / a.H);
  int tok0, L, srow0, sblk0;
  a.seq.get(s, tok0, L, srow0, sblk0);
  tok0 = __builtin_amdgcn_readfirstlane(tok0);
  L = __builtin_amdgcn_readfirstlane(L);
  const int qbase = qt * BM;
  if (qbase >= L) return;
  const int q0 = qbase + 32 * w;
  const int qi = q0 + n;
  const long rowH = (long)a.H * D;   // elements between consecutive tokens
  const uint16_t* gq = (const uint16_t*)a.q;
  const uint16_t* gk = (const uint16_t*)a.k;
  const uint16_t* gv = (const uint16_t*)a.v;

  // one 64-key tile: buffer resources end with the sequence, so rows past it read as zero
  auto load_tile = [&](int t, KVStage16<D>& st) {
    const int k0 = t * BN;
    const int rows = min(BN, L - k0);   // >= 1
    const long tb = (long)(tok0 + k0) * rowH + (long)h * D;
    const int nrec = ((rows - 1) * (int)rowH + D) * 2;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(gk + tb, nrec), rv = buffer_rsrc(gv + tb, nrec);
#pragma unroll
    for (int c = 0; c < KVStage16<D>::CH; ++c) {
      const int ch = tid + c * NT;
      const int off = (ch / CPR) * (int)rowH * 2 + (ch % CPR) * 16;
      st.k[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      st.v[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  };
  auto store_tile = [&](int buf, const KVStage16<D>& st) {
#pragma unroll
    for (int c = 0; c < KVStage16<D>::CH; ++c) {
      const int ch = tid + c * NT;
      const int r = ch / CPR, cx = ch % CPR;
      *(uint4*)(&sK[buf][r * KSK + cx * 16]) = st.k[c];
      *(uint4*)(&sV[buf][r * KSV + cx * 16]) = st.v[c];
    }
  };

  // ---- Q as the second operand, resident: qa[k] = features 16k + 8g + 0..7 of query qi
  uint4 qa[NK];
  if (qi < L) {
    const uint16_t* qp = gq + (long)(tok0 + qi) * rowH + (long)h * D;
#pragma unroll
    for (int k = 0; k < NK; ++k) qa[k] = *(const uint4*)(qp + 16 * k + 8 * g);
  } else {
#pragma unroll
    for (int k = 0; k < NK; ++k) qa[k] = make_uint4(0, 0, 0, 0);
  }

  const int kend = CAUSAL ? min(L, qbase + BM) : L;
  const int ntiles = (kend + BN - 1) / BN;

  v16f o[ND];
#pragma unroll
  for (int dc = 0; dc < ND; ++dc) o[dc] = v16f{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.c;

  {
    KVStage16<D> st0;
    load_tile(0, st0);
    store_tile(0, st0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BN;
    const int cur = t & 1;
    KVStage16<D> nxt;
    load_tile(min(t + 1, ntiles - 1), nxt);   // past the last tile, the last one again

    const bool compute = q0 < L && !(CAUSAL && k0 > q0 + 31);
    if (compute) {
      const uint8_t* sKc = sK[cur];
      const uint8_t* sVc = sV[cur];
      // ---- S^T = K Q^T: st[kb] element i holds key k0 + 32 kb + 8(i/4) + 4g + i%4, query qi
      v16f st[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint8_t* kp = sKc + (kb * 32 + n) * KSK + 16 * g;
        v16f acc = v16f{};
#pragma unroll
        for (int k = 0; k < NK; ++k) acc = mfma_bf16(as_v8bf(*(const uint4*)(kp + 32 * k)), as_v8bf(qa[k]), acc);
        st[kb] = acc;
      }
      const bool need_mask = (k0 + BN > L) || (CAUSAL && k0 + BN - 1 > q0);
      if (need_mask) {
        const int last = CAUSAL ? min(L - 1, qi) : L - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int hi = last - k0 - 32 * kb - 4 * g + 1;
#pragma unroll
          for (int i = 0; i < 16; ++i) st[kb][i] = (8 * (i >> 2) + (i & 3) < hi) ? st[kb][i] : -INFINITY;
        }
      }
      float mx = st[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = (kb == 0 ? 1 : 0); i < 16; ++i) mx = fmaxf(mx, st[kb][i]);
      mx = half_swap_max(mx);
      // lazy integer frame, as in the MXFP8 forward
      const float m_tile = ceilf(mx * c);
      if (m_tile > m_run + kLazy) {
        const float alpha = (m_run == -INFINITY) ? 0.f : ldexpf(1.f, (int)(m_run - m_tile));
#pragma unroll
        for (int dc = 0; dc < ND; ++dc) o[dc] *= alpha;
        l_run *= alpha;
        m_run = m_tile;
      }
      const float negM = -m_run;
      float psum = 0.f;
      // ---- p, running sum, bf16 pairs: pw[kb][q] = keys 8q + 4g + {0,1}, {2,3} of block kb
      uint32_t pw[2][4][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = __builtin_amdgcn_exp2f(fmaf(st[kb][4 * q + e], c, negM));
            psum += p[e];
          }
          pw[kb][q][0] = pack_bf16(p[0], p[1]);
          pw[kb][q][1] = pack_bf16(p[2], p[3]);
        }
      l_run += psum;
      // ---- regroup: for 16-key step ks = 2 kb + h2, lane half g holds keys 16 ks + 8g + 0..7
      uint4 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          auto s0 = __builtin_amdgcn_permlane32_swap(pw[kb][2 * h2][0], pw[kb][2 * h2 + 1][0], false, false);
          auto s1 = __builtin_amdgcn_permlane32_swap(pw[kb][2 * h2][1], pw[kb][2 * h2 + 1][1], false, false);
          pb[2 * kb + h2] = make_uint4(s0[0], s1[0], s0[1], s1[1]);
        }
      // ---- O^T += V^T P^T: lane (n, g) of step ks supplies V[keys 16 ks + 8g + 0..7][d = 32 dc + n]
      {
        const int G = lane >> 4, i16 = lane & 15;
        const int rowofs = 8 * g + (i16 >> 2);
        const int colb = 2 * (16 * (G & 1) + 4 * (i16 & 3));
#pragma unroll
        for (int dc = 0; dc < ND; ++dc)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) {
            const uint8_t* vp = sVc + (16 * ks + rowofs) * KSV + 64 * dc + colb;
            const uint2 r0 = lds_tr16(vp), r1 = lds_tr16(vp + 4 * KSV);
            o[dc] = mfma_bf16(as_v8bf(make_uint4(r0.x, r0.y, r1.x, r1.y)), as_v8bf(pb[ks]), o[dc]);
          }
      }
    }
    store_tile(cur ^ 1, nxt);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = ln2 (M + log2 l); each lane half summed its 16 keys per block
  l_run += __shfl_xor(l_run, 32, 64);
  if (qi >= L) return;
  const float inv = 1.f / l_run;
  const long orow = (long)(tok0 + qi) * rowH + (long)h * D;
#pragma unroll
  for (int dc = 0; dc < ND; ++dc)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * dc + 8 * q + 4 * g;
      const float v0 = o[dc][4 * q] * inv, v1 = o[dc][4 * q + 1] * inv, v2 = o[dc][4 * q + 2] * inv,
                  v3 = o[dc][4 * q + 3] * inv;
      if constexpr (OUT_BF16) {
        uint2 pk = make_uint2(f32_to_bf16(v0) | (f32_to_bf16(v1) << 16), f32_to_bf16(v2) | (f32_to_bf16(v3) << 16));
        *(uint2*)((uint16_t*)a.o + orow + d) = pk;
      } else {
        *(float4*)((float*)a.o + orow + d) = make_float4(v0, v1, v2, v3);
      }
    }
  if (g == 0 && a.lse) {
    const long li = a.seq.cu ? (long)h * a.T + tok0 + qi : ((long)s * a.H + h) * a.seq.S + qi;
    a.lse[li] = 0.69314718055994531f * (m_run + log2f(l_run));
  }
}

hipError_t launch_attn_fwd_bf16(int D, bool causal, bool out_bf16, FwdArgs a, int max_len, hipStream_t st) {
  constexpr int NW = 4;
  a.nqt = (max_len + 32 * NW - 1) / (32 * NW);
  const long units = (long)a.nseq * a.H;
  const long grid = ((units + 7) / 8) * 8 * a.nqt;
  if (grid == 0) return hipSuccess;
  dim3 g((unsigned)grid), b(NW * 64);
#define MX_FWD16_CASE(DD, CC, OB) \
  if (D == DD && causal == CC && out_bf16 == OB) { attn_fwd_bf16_kernel<DD, CC, OB><<<g, b, 0, st>>>(a); return hipGetLastError(); }
  MX_FWD16_CASE(64, false, false) MX_FWD16_CASE(64, false, true) MX_FWD16_CASE(64, true, false) MX_FWD16_CASE(64, true, true)
  MX_FWD16_CASE(128, false, false) MX_FWD16_CASE(128, false, true) MX_FWD16_CASE(128, true, false) MX_FWD16_CASE(128, true, true)
#undef MX_FWD16_CASE
  return hipErrorInvalidValue;
}

}  // namespace mxk
