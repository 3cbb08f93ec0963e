// Fused MXFP8 attention backward for gfx950.
//
// What is computed follows "Low Precision Flash Attention 4: End-to-End
// Block-Scaled Attention for Blackwell": the forward/backward paragraph (Q,
// K and dO quantized in square [32, 32] blocks so one payload serves both
// orientations; P recomputed; dQ reduced in FP16 under a static power-of-two
// scale) and the contributions paragraph (dS quantized online in
// transpose-invariant square blocks); and "Low-Precision FlashAttention-4 ...
// for NVIDIA Blackwell", section "3. Gradient Scale Recomputation in the
// Backward Pass" (MX scales of the gradients recomputed inside the kernel).
//
// Three kernels on the caller's stream:
//  1. bwd_pre_kernel: D_i = sum_d dO_id O_id in fp32 from the unquantized
//     tensors, and zero the fp16 dQ accumulator.
//  2. attn_bwd_kernel: one workgroup per (sequence, head, 128-key tile),
//     four waves of 32 keys, walking 64-query tiles.  Per tile each wave
//     computes S = Q^ K^T and dP = dO^ V^T (scaled MFMA, keys as the output
//     columns so a lane owns one key), p = exp2(S c - LSE log2 e),
//     dS = p (dP - D), then MX codes of P (32 queries per key) and of dS
//     (square 32 x 32 blocks, wave-wide amax), and accumulates dV^T and
//     dK^T in registers.  The dS codes go to LDS, and the workgroup's waves
//     then form dQ = dS K for the tile (128 keys of contraction) and add it,
//     scaled by softmax_scale * 2^s, into the fp16 accumulator with packed
//     fp16 atomics laid along contiguous features (neighbouring lanes pair
//     up), so each atomic instruction touches four 64-byte row segments.  Q^ and dO^ are read from LDS in both
//     orientations: rows as MFMA operands, columns through
//     ds_read_b64_tr_b8 (one payload, both GEMMs).
//  3. bwd_dq_kernel: dQ = acc * 2^-s in the output type.
#include "mx_common.h"
#include "mx_launch.h"

namespace mxk {

namespace {

template <int OA, int OB>
MX_DEV v16f mfma32b(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OA, sa, OB, sb);
}

MX_DEV v8i pack8b(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

MX_DEV v2i tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((v2i __attribute__((address_space(3)))*)(p));
}

// 64-deep operand whose K index runs down rows `row0 + {0..15}` (block 0) and
// `row0 + 32 + {0..15}` (block 1) of a row-major byte tile, lane column
// `col0 + lane % 32`: four transpose reads.
MX_DEV v8i tr_operand(const uint8_t* base, int stride, int lane) {
  const int G = lane >> 4, i16 = lane & 15;
  const uint8_t* p = base + (16 * (G >> 1) + (i16 >> 1)) * stride + 16 * (G & 1) + 8 * (i16 & 1);
  v2i r0 = tr8(p), r1 = tr8(p + 8 * stride), r2 = tr8(p + 32 * stride), r3 = tr8(p + 40 * stride);
  return v8i{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

MX_DEV uint32_t ld_scale_word(const uint8_t* p, int nbytes) {
  return nbytes == 4 ? *(const uint32_t*)p : *(const uint16_t*)p;
}

MX_DEV float wave_max_all(float v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

MX_DEV void atomic_add_h2(_Float16* p, float a, float b) {
  h2v v = {(_Float16)a, (_Float16)b};
  __builtin_amdgcn_global_atomic_fadd_v2f16((h2v __attribute__((address_space(1)))*)(p), v);
}

}  // namespace

// ------------------------------------------------------------ preprocess
template <int D, bool F32>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int EPC = F32 ? 4 : 8;       // elements per 16-byte chunk
  constexpr int LPR = D / EPC;           // lanes per row
  constexpr int RPW = 64 / LPR;          // rows per wave
  const int lane = threadIdx.x & 63;
  const long wave = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long row = wave * RPW + lane / LPR;        // global (token, head) row
  const long nrows = (long)a.T * a.H;
  const int c = lane % LPR;
  float acc = 0.f;
  if (row < nrows) {
    const long off = row * D + c * EPC;
    if constexpr (F32) {
      float4 x = *(const float4*)((const float*)a.o + off);
      float4 y = *(const float4*)((const float*)a.dout + off);
      acc = x.x * y.x + x.y * y.y + x.z * y.z + x.w * y.w;
    } else {
      uint4 x = *(const uint4*)((const uint16_t*)a.o + off);
      uint4 y = *(const uint4*)((const uint16_t*)a.dout + off);
      acc = bf16_lo(x.x) * bf16_lo(y.x) + bf16_hi(x.x) * bf16_hi(y.x) + bf16_lo(x.y) * bf16_lo(y.y) +
            bf16_hi(x.y) * bf16_hi(y.y) + bf16_lo(x.z) * bf16_lo(y.z) + bf16_hi(x.z) * bf16_hi(y.z) +
            bf16_lo(x.w) * bf16_lo(y.w) + bf16_hi(x.w) * bf16_hi(y.w);
    }
    // zero this row's fp16 dQ accumulator (D halves)
    uint4 z = make_uint4(0, 0, 0, 0);
    uint16_t* accp = (uint16_t*)a.acc + row * D;
    for (int i = c; i < D / 8; i += LPR) *(uint4*)(accp + i * 8) = z;
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o, 64);
  if (row < nrows && c == 0) {
    const long tok = row / a.H;
    const int h = (int)(row % a.H);
    long di;
    if (a.seq.cu) di = (long)h * a.T + tok;
    else di = ((tok / a.seq.S) * a.H + h) * (long)a.seq.S + tok % a.seq.S;
    a.Dbuf[di] = acc;
  }
}

// ------------------------------------------------------------ main kernel
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_bwd_kernel(BwdArgs a) {
  constexpr int BN = 32 * NW;   // keys per workgroup
  constexpr int BQ = 64;        // queries per step
  constexpr int NC = D / 64;    // 64-feature chunks of the S / dP contraction
  constexpr int ND = D / 32;    // 32-feature chunks of dK, dV, dQ
  constexpr int NB = D / 32;    // scale bytes per SQ32 / ROW32 scale word
  constexpr int KST = D + 16;   // LDS row stride of K, Q, dO tiles
  constexpr int SST = BQ + 16;  // LDS row stride of the dS code tile [key][query]
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) uint8_t sK[BN * KST];
  __shared__ __attribute__((aligned(16))) uint8_t sQ[BQ * KST];
  __shared__ __attribute__((aligned(16))) uint8_t sDO[BQ * KST];
  __shared__ __attribute__((aligned(16))) uint8_t sDS[BN * SST];
  __shared__ uint32_t sKs[NW];       // K SQ32 scale word (bytes = feature blocks) per key block
  __shared__ uint32_t sQs[2], sDOs[2];
  __shared__ uint32_t sDSs[2][NW];   // dS scale of (query block t, key block)
  __shared__ float sL[BQ], sDv[BQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, n = lane & 31;
  const int id = blockIdx.x, xcd = id & 7, jj = id >> 3;
  const int u = (jj / a.nkt) * 8 + xcd;
  if (u >= a.nseq * a.H) return;
  const int kt = jj % a.nkt;          // low key tiles see the most queries under causality: first
  const int h = u % a.H, s = u / a.H;
  int tok0, L, srow0, sblk0;
  a.seq.get(s, tok0, L, srow0, sblk0);
  const int kbase = kt * BN;
  if (kbase >= L) return;
  const long rowH = (long)a.H * D;
  const int kw0 = kbase + 32 * w;
  const int kj = kw0 + n;

  // ---- K tile (all keys of the workgroup) for the dQ products, and scales
  for (int ch = tid; ch < BN * D / 16; ch += NT) {
    const int r = ch / (D / 16), cx = ch % (D / 16);
    uint4 kv = make_uint4(0, 0, 0, 0);
    if (kbase + r < L) kv = *(const uint4*)(a.k + (long)(tok0 + kbase + r) * rowH + (long)h * D + cx * 16);
    *(uint4*)(sK + r * KST + cx * 16) = kv;
  }
  if (tid < NW) {
    uint32_t wk = 0;
    if (kbase + 32 * tid < L)
      wk = ld_scale_word(a.ks + ((long)(sblk0 + kbase / 32 + tid) * a.H + h) * NB, NB);
    sKs[tid] = wk;
  }
  // ---- this wave's keys as the column operand of S = Q K^T and dP = dO V^T
  v8i kb[NC], vb[NC];
  uint32_t ksc = 0, vsc = 0;
  if (kj < L) {
    const uint8_t* kp = a.k + (long)(tok0 + kj) * rowH + (long)h * D;
    const uint8_t* vp = a.v + (long)(tok0 + kj) * rowH + (long)h * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kb[c] = pack8b(*(const uint4*)(kp + 64 * c + 16 * g), *(const uint4*)(kp + 64 * c + 32 + 16 * g));
      vb[c] = pack8b(*(const uint4*)(vp + 64 * c + 16 * g), *(const uint4*)(vp + 64 * c + 32 + 16 * g));
    }
    ksc = ld_scale_word(a.ks + ((long)(sblk0 + kw0 / 32) * a.H + h) * NB, NB) >> (8 * g);
    vsc = ld_scale_word(a.vs + ((long)(srow0 + kj) * a.H + h) * NB, NB) >> (8 * g);
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kb[c] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      vb[c] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  v16f dvt[ND], dkt[ND];   // dV^T, dK^T: element i = feature 32 dc + 8(i/4) + 4g + i%4, key kj
#pragma unroll
  for (int dc = 0; dc < ND; ++dc) {
    dvt[dc] = v16f{};
    dkt[dc] = v16f{};
  }
  const float c = a.c;
  const int qstart = CAUSAL ? (kbase / BQ) * BQ : 0;
  // scale operands of the last dV / dK products, pinned until those products finish
  uint32_t dosw_prev = 0, qsw_prev = 0;
  int psc_prev = 0, ssc_prev = 0;

  for (int q0 = qstart; q0 < L; q0 += BQ) {
    __syncthreads();
    // ---- stage the Q and dO tiles, their scales, LSE*log2(e) and D
    for (int ch = tid; ch < BQ * D / 16; ch += NT) {
      const int r = ch / (D / 16), cx = ch % (D / 16);
      uint4 qv = make_uint4(0, 0, 0, 0), dv = make_uint4(0, 0, 0, 0);
      if (q0 + r < L) {
        const long off = (long)(tok0 + q0 + r) * rowH + (long)h * D + cx * 16;
        qv = *(const uint4*)(a.q + off);
        dv = *(const uint4*)(a.dob + off);
      }
      *(uint4*)(sQ + r * KST + cx * 16) = qv;
      *(uint4*)(sDO + r * KST + cx * 16) = dv;
    }
    if (tid < 2) {
      uint32_t wq = 0, wd = 0;
      if (q0 + 32 * tid < L) {
        const long so = ((long)(sblk0 + q0 / 32 + tid) * a.H + h) * NB;
        wq = ld_scale_word(a.qs + so, NB);
        wd = ld_scale_word(a.dos + so, NB);
      }
      sQs[tid] = wq;
      sDOs[tid] = wd;
    }
    for (int r = tid; r < BQ; r += NT) {
      float l2 = 0.f, dd = 0.f;
      if (q0 + r < L) {
        const long li = a.seq.cu ? (long)h * a.T + tok0 + q0 + r : ((long)s * a.H + h) * a.seq.S + q0 + r;
        l2 = a.lse[li] * 1.44269504088896340736f;
        dd = a.Dbuf[li];
      }
      sL[r] = l2;
      sDv[r] = dd;
    }
    __syncthreads();

    const bool active = kw0 < L && !(CAUSAL && kw0 > q0 + BQ - 1);
    if (active) {
      // ---- S and dP for two 32-query blocks: element i = query q0 + 32t + 8(i/4) + 4g + i%4, key kj
      v16f st[2], dpt[2];
      uint32_t qsa[2], dsa[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const uint8_t* qp = sQ + (32 * t + n) * KST + 16 * g;
        const uint8_t* op = sDO + (32 * t + n) * KST + 16 * g;
        qsa[t] = sQs[t] >> (8 * g);
        dsa[t] = sDOs[t] >> (8 * g);
        v16f sa = v16f{}, da = v16f{};
        sa = mfma32b<0, 0>(pack8b(*(const uint4*)qp, *(const uint4*)(qp + 32)), kb[0], sa, qsa[t], ksc);
        da = mfma32b<0, 0>(pack8b(*(const uint4*)op, *(const uint4*)(op + 32)), vb[0], da, dsa[t], vsc);
        if constexpr (NC > 1) {
          sa = mfma32b<2, 2>(pack8b(*(const uint4*)(qp + 64), *(const uint4*)(qp + 96)), kb[NC - 1], sa, qsa[t], ksc);
          da = mfma32b<2, 2>(pack8b(*(const uint4*)(op + 64), *(const uint4*)(op + 96)), vb[NC - 1], da, dsa[t], vsc);
        }
        st[t] = sa;
        dpt[t] = da;
      }
      // ---- p = 2^(S c - LSE log2 e) (0 where masked), dS = p (dP - D)
      float amax[2], smax[2];   // largest exp2 argument of each P block; |dS| max of each dS block
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float am = -INFINITY, sm = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int ql = 32 * t + 8 * (i >> 2) + 4 * g + (i & 3);
          const int qi = q0 + ql;
          const bool masked = qi >= L || kj >= L || (CAUSAL && kj > qi);
          const float arg = masked ? -INFINITY : fmaf(st[t][i], c, -sL[ql]);
          const float p = __builtin_amdgcn_exp2f(arg);
          const float ds = p * (dpt[t][i] - sDv[ql]);
          st[t][i] = p;
          dpt[t][i] = ds;
          am = fmaxf(am, arg);
          sm = fmaxf(sm, fabsf(ds));
        }
        amax[t] = fmaxf(am, __shfl_xor(am, 32, 64));   // 32 queries of this key
        smax[t] = wave_max_all(sm);                      // 32 queries x 32 keys
      }
      // S and dP have been read: their products and the previous step's dV, dK products are done
      keep(qsa[0]); keep(qsa[1]); keep(dsa[0]); keep(dsa[1]);
      keep(dosw_prev); keep(qsw_prev); keep(psc_prev); keep(ssc_prev);
      // ---- MX codes: dword q of block t holds queries 8q + 4g + 0..3
      uint32_t pw[2][4], sw[2][4];
      int kp[2], ks2[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        kp[t] = max(exp2_scale_code(amax[t]), 1);
        ks2[t] = max(scale_code(smax[t]), 1);
        const float psc = e8m0_f32(kp[t]), plim = 448.f * psc;
        const float ssc = e8m0_f32(ks2[t]), slim = 448.f * ssc;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v2s z = {0, 0};
          z = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, fminf(st[t][4 * q], plim), fminf(st[t][4 * q + 1], plim), psc,
                                                       false);
          z = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, fminf(st[t][4 * q + 2], plim), fminf(st[t][4 * q + 3], plim),
                                                       psc, true);
          pw[t][q] = __builtin_bit_cast(uint32_t, z);
          v2s y = {0, 0};
          y = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(y, __builtin_amdgcn_fmed3f(dpt[t][4 * q], -slim, slim),
                                                       __builtin_amdgcn_fmed3f(dpt[t][4 * q + 1], -slim, slim), ssc,
                                                       false);
          y = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(y, __builtin_amdgcn_fmed3f(dpt[t][4 * q + 2], -slim, slim),
                                                       __builtin_amdgcn_fmed3f(dpt[t][4 * q + 3], -slim, slim), ssc,
                                                       true);
          sw[t][q] = __builtin_bit_cast(uint32_t, y);
          // dS codes to LDS as [key][query] for the dQ products
          *(uint32_t*)(sDS + (32 * w + n) * SST + 32 * t + 8 * q + 4 * g) = sw[t][q];
        }
      }
      if (lane == 0) {
        sDSs[0][w] = ks2[0];
        sDSs[1][w] = ks2[1];
      }
      // ---- swap lane halves: half g then holds queries 16g + 0..15 of each block, in order
      v8i pP, pS;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        auto a02 = __builtin_amdgcn_permlane32_swap(pw[t][0], pw[t][2], false, false);
        auto a13 = __builtin_amdgcn_permlane32_swap(pw[t][1], pw[t][3], false, false);
        pP[4 * t + 0] = a02[0]; pP[4 * t + 1] = a02[1]; pP[4 * t + 2] = a13[0]; pP[4 * t + 3] = a13[1];
        auto b02 = __builtin_amdgcn_permlane32_swap(sw[t][0], sw[t][2], false, false);
        auto b13 = __builtin_amdgcn_permlane32_swap(sw[t][1], sw[t][3], false, false);
        pS[4 * t + 0] = b02[0]; pS[4 * t + 1] = b02[1]; pS[4 * t + 2] = b13[0]; pS[4 * t + 3] = b13[1];
      }
      const int pscale = g ? kp[1] : kp[0];
      const int sscale = g ? ks2[1] : ks2[0];
      const uint32_t dosw = sDOs[g], qsw = sQs[g];
      dosw_prev = dosw; qsw_prev = qsw; psc_prev = pscale; ssc_prev = sscale;
      // ---- dV^T += dO^T P^ and dK^T += Q^T dS^ (rows: features, contraction: the 64 queries)
#pragma unroll
      for (int dc = 0; dc < ND; ++dc) {
        const v8i oa = tr_operand(sDO + 32 * dc, KST, lane);
        const v8i qa = tr_operand(sQ + 32 * dc, KST, lane);
        if (dc == 0) { dvt[0] = mfma32b<0, 0>(oa, pP, dvt[0], dosw, pscale); dkt[0] = mfma32b<0, 0>(qa, pS, dkt[0], qsw, sscale); }
        if (dc == 1) { dvt[1] = mfma32b<1, 0>(oa, pP, dvt[1], dosw, pscale); dkt[1] = mfma32b<1, 0>(qa, pS, dkt[1], qsw, sscale); }
        if constexpr (ND > 2) {
          if (dc == 2) { dvt[2] = mfma32b<2, 0>(oa, pP, dvt[2], dosw, pscale); dkt[2] = mfma32b<2, 0>(qa, pS, dkt[2], qsw, sscale); }
          if (dc == 3) { dvt[3] = mfma32b<3, 0>(oa, pP, dvt[3], dosw, pscale); dkt[3] = mfma32b<3, 0>(qa, pS, dkt[3], qsw, sscale); }
        }
      }
    } else {
      // keys entirely after this query tile (or past the sequence): their dS is zero
      const uint4 z = make_uint4(0, 0, 0, 0);
      uint8_t* rowp = sDS + (32 * w + (lane >> 1)) * SST + 32 * (lane & 1);
      *(uint4*)rowp = z;
      *(uint4*)(rowp + 16) = z;
      if (lane == 0) {
        sDSs[0][w] = 0;
        sDSs[1][w] = 0;
      }
    }
    __syncthreads();

    // ---- dQ for (query block t, feature chunk dc) pairs, shared out among the waves.
    // Output element i of lane l: query 32t + 8(i/4) + 4g + i%4, feature 32 dc + l%32, so a
    // wave's atomics run along contiguous features of a few query rows.
    for (int cb = w; cb < 2 * ND; cb += NW) {
      const int t = cb / ND, dc = cb % ND;
      if (q0 + 32 * t >= L) continue;
      v16f acc = v16f{};
      v8i ka[BN / 64], sb[BN / 64];
      int kscale[BN / 64], sscale[BN / 64];
#pragma unroll
      for (int kk = 0; kk < BN / 64; ++kk) {
        sb[kk] = tr_operand(sDS + (64 * kk) * SST + 32 * t, SST, lane);   // rows: queries, K: keys
        ka[kk] = tr_operand(sK + (64 * kk) * KST + 32 * dc, KST, lane);   // columns: features, K: keys
        sscale[kk] = (int)sDSs[t][2 * kk + g];
        kscale[kk] = (int)((sKs[2 * kk + g] >> (8 * dc)) & 0xFFu);
        if (CAUSAL && kbase + 64 * kk > q0 + 32 * t + 31) continue;   // every key after every query
        acc = mfma32b<0, 0>(sb[kk], ka[kk], acc, sscale[kk], kscale[kk]);
      }
      keep(acc[0]);
#pragma unroll
      for (int kk = 0; kk < BN / 64; ++kk) {
        keep(kscale[kk]);
        keep(sscale[kk]);
      }
      // pair neighbouring lanes: the even lane of a pair adds (row, f..f+1) of element i, the
      // odd lane (row + 1, f-1..f) of element i + 1
      const bool odd = lane & 1;
      const int fcol = 32 * dc + n - (odd ? 1 : 0);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float mine = odd ? acc[i + 1] : acc[i];
        const float send = odd ? acc[i] : acc[i + 1];
        const float got = __shfl_xor(send, 1, 64);
        const int ql = 32 * t + 8 * (i >> 2) + 4 * g + (i & 3) + (odd ? 1 : 0);
        const int qi = q0 + ql;
        if (qi < L) {
          _Float16* ap = (_Float16*)a.acc + (long)(tok0 + qi) * rowH + (long)h * D + fcol;
          if (odd) atomic_add_h2(ap, got * a.dq_mult, mine * a.dq_mult);
          else atomic_add_h2(ap, mine * a.dq_mult, got * a.dq_mult);
        }
      }
    }
  }

  // ---- epilogue: dK = softmax_scale * dK^T, dV = dV^T, features 32 dc + 8q + 4g + 0..3 of key kj
  keep(dvt[ND - 1][0]);
  keep(dkt[ND - 1][0]);
  keep(dosw_prev); keep(qsw_prev); keep(psc_prev); keep(ssc_prev);
  if (kj >= L) return;
  const long orow = (long)(tok0 + kj) * rowH + (long)h * D;
#pragma unroll
  for (int dc = 0; dc < ND; ++dc)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * dc + 8 * q + 4 * g;
      const float k0 = dkt[dc][4 * q] * a.sigma, k1 = dkt[dc][4 * q + 1] * a.sigma, k2 = dkt[dc][4 * q + 2] * a.sigma,
                  k3 = dkt[dc][4 * q + 3] * a.sigma;
      const float v0 = dvt[dc][4 * q], v1 = dvt[dc][4 * q + 1], v2 = dvt[dc][4 * q + 2], v3 = dvt[dc][4 * q + 3];
      if (a.grad_f32) {
        *(float4*)((float*)a.dk + orow + d) = make_float4(k0, k1, k2, k3);
        *(float4*)((float*)a.dv + orow + d) = make_float4(v0, v1, v2, v3);
      } else {
        *(uint2*)((uint16_t*)a.dk + orow + d) =
            make_uint2(f32_to_bf16(k0) | (f32_to_bf16(k1) << 16), f32_to_bf16(k2) | (f32_to_bf16(k3) << 16));
        *(uint2*)((uint16_t*)a.dv + orow + d) =
            make_uint2(f32_to_bf16(v0) | (f32_to_bf16(v1) << 16), f32_to_bf16(v2) | (f32_to_bf16(v3) << 16));
      }
    }
}

// ------------------------------------------------------------ dQ finalize
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 raw = *((const uint4*)a.acc + i);
  const _Float16* hp = (const _Float16*)&raw;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (float)hp[e] * a.dq_unscale;
  if (a.grad_f32) {
    float4* o = (float4*)a.dq + 2 * i;
    o[0] = make_float4(v[0], v[1], v[2], v[3]);
    o[1] = make_float4(v[4], v[5], v[6], v[7]);
  } else {
    uint4 o;
    o.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    o.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
    o.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
    o.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
    *((uint4*)a.dq + i) = o;
  }
}

template __global__ void attn_bwd_kernel<64, 4, true>(BwdArgs);
template __global__ void attn_bwd_kernel<64, 4, false>(BwdArgs);
template __global__ void attn_bwd_kernel<128, 4, true>(BwdArgs);
template __global__ void attn_bwd_kernel<128, 4, false>(BwdArgs);

hipError_t launch_attn_bwd(int D, bool causal, bool io_f32, BwdArgs a, int max_len, hipStream_t st) {
  constexpr int NW = 4;
  const long rows = (long)a.T * a.H;
  if (rows == 0) return hipSuccess;
  // 1. D_i and zeroed accumulator
  {
    const int epc = io_f32 ? 4 : 8;
    const int rpw = 64 / (D / epc);
    const long waves = (rows + rpw - 1) / rpw;
    dim3 g((unsigned)((waves + 3) / 4)), b(256);
    if (D == 64 && !io_f32) bwd_pre_kernel<64, false><<<g, b, 0, st>>>(a);
    else if (D == 64) bwd_pre_kernel<64, true><<<g, b, 0, st>>>(a);
    else if (!io_f32) bwd_pre_kernel<128, false><<<g, b, 0, st>>>(a);
    else bwd_pre_kernel<128, true><<<g, b, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // 2. main
  {
    a.nkt = (max_len + 32 * NW - 1) / (32 * NW);
    const long units = (long)a.nseq * a.H;
    const long grid = ((units + 7) / 8) * 8 * a.nkt;
    dim3 g((unsigned)grid), b(NW * 64);
    if (D == 64 && causal) attn_bwd_kernel<64, NW, true><<<g, b, 0, st>>>(a);
    else if (D == 64) attn_bwd_kernel<64, NW, false><<<g, b, 0, st>>>(a);
    else if (causal) attn_bwd_kernel<128, NW, true><<<g, b, 0, st>>>(a);
    else attn_bwd_kernel<128, NW, false><<<g, b, 0, st>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // 3. dQ = acc * 2^-s
  {
    const long n8 = rows * D / 8;
    dim3 g((unsigned)((n8 + 255) / 256)), b(256);
    bwd_dq_kernel<<<g, b, 0, st>>>(a, n8);
    return hipGetLastError();
  }
}

}  // namespace mxk
