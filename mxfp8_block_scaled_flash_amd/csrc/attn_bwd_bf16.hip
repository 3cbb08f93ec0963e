// BF16 attention backward for gfx950: the baseline of the MXFP8 backward
// ("Low Precision Flash Attention 4: End-to-End Block-Scaled Attention for
// Blackwell", headline speed-ups over BF16 FlashAttention-4).
//
// Same computation as the MXFP8 backward with every MX step removed: S and dP
// from bf16 operands in fp32, p = 2^(S c - LSE log2 e), D_i = rowsum(dO o O)
// in fp32, dS = p (dP - D), P and dS rounded to bf16 (nearest even) for
// dV = P^T dO, dK = sigma dS^T Q and dQ = sigma dS K.
//
// gfx950 design.  Device-scope atomics execute at the memory side on this
// chip (the per-XCD L2s are not coherent with each other), and an fp32 dQ
// reduction over 128-key tiles would move about four times the MXFP8
// backward's atomic traffic (fp16 atomics alone over 128-key tiles took
// 14 ms).  So dQ is not reduced with atomics:
//  1. bwd_pre_kernel (shared with the MXFP8 path): D_i.
//  2. dkdv kernel, key-stationary: a workgroup of 8 waves (two per SIMD) owns
//     128 keys held in LDS; wave w takes key block w % 4 and query block
//     w / 4 of every 64-query step (Q, dO, LSE, D double-buffered in LDS),
//     computes S = Q K^T and dP = dO V^T with keys as the output columns (a
//     lane owns one key), and accumulates dV^T += dO^T P and dK^T += Q^T dS
//     in registers, the transposed Q and dO operands read with
//     ds_read_b64_tr_b16; the two waves of a key block add their partials
//     through LDS at the end.
//  3. dq kernel, query-stationary (the forward's skeleton): a wave owns 32
//     queries with Q and dO resident, walks 64-key tiles of K and V staged in
//     LDS, recomputes S^T and dP^T, and accumulates dQ^T += K^T dS^T in
//     registers; one write per element, no reduction across workgroups.
// The recompute costs three extra products per pair (7 instead of 5), in
// exchange for no atomics and a deterministic result.
#include "mx_common.h"
#include "mx_launch.h"

namespace mxk {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));

MX_DEV v16f mfma_bf16(uint4 a, uint4 b, const v16f& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
}

MX_DEV uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{a, b}, v2bf));
}

MX_DEV uint2 lds_tr16(const uint8_t* p) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((v4s __attribute__((address_space(3)))*)(p)));
}

// Transposed operand from a row-major bf16 tile with row stride RS bytes: lane (n, g) receives
// element (rows r0 + 8g + 0..7, column c0 + n), i.e. 8 consecutive rows of one column.  In each
// 16-lane group G, lane i addresses row r0 + 8g + 4h + i/4 at column c0 + 16(G%2) + 4(i%4) for
// the h-th read, and receives column c0 + 16(G%2) + i of the four rows read by lanes i/4 + 4m.
template <int RS>
MX_DEV uint4 tr_operand(const uint8_t* tile, int r0, int c0, int lane) {
  const int G = lane >> 4, i16 = lane & 15, g = lane >> 5;
  const uint8_t* p = tile + (r0 + 8 * g + (i16 >> 2)) * RS + 2 * (c0 + 16 * (G & 1) + 4 * (i16 & 3));
  const uint2 a = lds_tr16(p), b = lds_tr16(p + 4 * RS);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// Regroup 16 fp32 values held in the 32x32 output layout (element i = row 8(i/4) + 4g + i%4 of
// the block) into bf16 operands: op[h] holds rows 16h + 8g + 0..7 of the block, in order.
MX_DEV void to_operands(const float* x, uint4 op[2]) {
  uint32_t w[4][2];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    w[q][0] = pack_bf16(x[4 * q], x[4 * q + 1]);
    w[q][1] = pack_bf16(x[4 * q + 2], x[4 * q + 3]);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    auto s0 = __builtin_amdgcn_permlane32_swap(w[2 * h][0], w[2 * h + 1][0], false, false);
    auto s1 = __builtin_amdgcn_permlane32_swap(w[2 * h][1], w[2 * h + 1][1], false, false);
    op[h] = make_uint4(s0[0], s1[0], s0[1], s1[1]);
  }
}

// store 4 consecutive values of one row, bf16 or fp32
MX_DEV void store4(void* base, long off, bool f32, float v0, float v1, float v2, float v3) {
  if (f32) {
    *(float4*)((float*)base + off) = make_float4(v0, v1, v2, v3);
  } else {
    *(uint2*)((uint16_t*)base + off) =
        make_uint2(f32_to_bf16(v0) | (f32_to_bf16(v1) << 16), f32_to_bf16(v2) | (f32_to_bf16(v3) << 16));
  }
}

}  // namespace

// ------------------------------------------------------------- dK, dV
// 8 waves per workgroup of 128 keys (two per SIMD): wave w owns key block w % 4 for query block
// w / 4 of every 64-query step, so the two waves of a key block split each step's queries and
// add their partial dK, dV through LDS at the end.  K, V (the workgroup's 128 rows) and the
// step's Q, dO, LSE, D sit in LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_bwd_bf16_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 8;
  constexpr int BN = 128;       // keys per workgroup (4 key blocks of 32)
  constexpr int BQ = 64;        // queries per step (2 query blocks of 32)
  constexpr int NK = D / 16;    // 16-feature steps of the S and dP contractions
  constexpr int ND = D / 32;    // 32-feature chunks of dK, dV
  constexpr int RB = 2 * D;     // bytes per token row of one head
  constexpr int RS = RB + 32;   // LDS row stride
  constexpr int CPR = RB / 16;
  constexpr int NT = NW * 64;
  constexpr int TILE_K = BN * RS, TILE_Q = BQ * RS;
  constexpr int SMEM = 2 * TILE_K + 4 * TILE_Q;   // K, V, Q[2], dO[2]; reused for the final reduction
  static_assert(SMEM >= 4 * 2 * ND * 16 * 64 * 4, "the partial dK, dV of four waves fit in the tiles");
  __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM];
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];   // fl32(LSE log2 e)
  __shared__ __attribute__((aligned(16))) float sD[2][BQ];   // D_i
  uint8_t* const sK = smem;
  uint8_t* const sV = smem + TILE_K;
  uint8_t* const sQ0 = smem + 2 * TILE_K;   // sQ[buf] = sQ0 + buf * TILE_Q
  uint8_t* const sO0 = smem + 2 * TILE_K + 2 * TILE_Q;

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = w & 3, qb = w >> 2;
  const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
  const int u = (j / a.nkt) * 8 + xcd;
  if (u >= a.nseq * a.H) return;
  const int kt = j % a.nkt;   // causal: the first key tiles have the most queries, so they go first
  const int h = __builtin_amdgcn_readfirstlane(u % a.H), s = __builtin_amdgcn_readfirstlane(u / a.H);
  int tok0, L, srow0, sblk0;
  a.seq.get(s, tok0, L, srow0, sblk0);
  tok0 = __builtin_amdgcn_readfirstlane(tok0);
  L = __builtin_amdgcn_readfirstlane(L);
  const int k0 = kt * BN;
  if (k0 >= L) return;
  const int kw0 = k0 + 32 * kb;   // this wave's first key
  const int key = kw0 + n;
  const long rowH = (long)a.H * D;
  const uint16_t *gq = (const uint16_t*)a.q, *gk = (const uint16_t*)a.k, *gv = (const uint16_t*)a.v;
  const uint16_t* gd = (const uint16_t*)a.dout;

  // ---- K and V rows of the workgroup (zero past the end)
  {
    const int rows = min(BN, L - k0);
    const long tb = (long)(tok0 + k0) * rowH + (long)h * D;
    const int nrec = ((rows - 1) * (int)rowH + D) * 2;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(gk + tb, nrec), rv = buffer_rsrc(gv + tb, nrec);
    for (int ch = tid; ch < BN * CPR; ch += NT) {
      const int off = (ch / CPR) * (int)rowH * 2 + (ch % CPR) * 16;
      const uint4 kv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      const uint4 vv = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
      *(uint4*)(sK + (ch / CPR) * RS + (ch % CPR) * 16) = kv;
      *(uint4*)(sV + (ch / CPR) * RS + (ch % CPR) * 16) = vv;
    }
  }

  const int qstart = CAUSAL ? (k0 / BQ) * BQ : 0;
  const int nsteps = (L - qstart + BQ - 1) / BQ;
  const float c = a.c;
  constexpr int CH = BQ * CPR / NT;   // 16-byte chunks per thread per tensor and step
  struct Step {
    uint4 q[CH], d[CH];
    float x;   // LSE (threads 0..63) or D (threads 64..127)
  };
  auto load_step = [&](int t, Step& st) {
    const int q0 = qstart + t * BQ;
    const int rows = min(BQ, L - q0);
    const long tb = (long)(tok0 + q0) * rowH + (long)h * D;
    const int nrec = ((rows - 1) * (int)rowH + D) * 2;
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(gq + tb, nrec), rd = buffer_rsrc(gd + tb, nrec);
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const int ch = tid + cc * NT;
      const int off = (ch / CPR) * (int)rowH * 2 + (ch % CPR) * 16;
      st.q[cc] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0));
      st.d[cc] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rd, off, 0, 0));
    }
    const long li = a.seq.cu ? (long)h * a.T + tok0 + q0 : ((long)s * a.H + h) * a.seq.S + q0;
    const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(a.lse + li, rows * 4), rD = buffer_rsrc(a.Dbuf + li, rows * 4);
    st.x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(w == 0 ? rl : rD, lane * 4, 0, 0));
  };
  auto store_step = [&](int buf, const Step& st) {
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
      const int ch = tid + cc * NT;
      const int r = ch / CPR, cx = ch % CPR;
      *(uint4*)(sQ0 + buf * TILE_Q + r * RS + cx * 16) = st.q[cc];
      *(uint4*)(sO0 + buf * TILE_Q + r * RS + cx * 16) = st.d[cc];
    }
    if (w == 0) sL[buf][lane] = st.x * 1.44269504088896340736f;
    else if (w == 1) sD[buf][lane] = st.x;
  };

  v16f dk[ND], dv[ND];
#pragma unroll
  for (int dc = 0; dc < ND; ++dc) dk[dc] = dv[dc] = v16f{};

  {
    Step s0;
    load_step(0, s0);
    store_step(0, s0);
  }
  __syncthreads();

  for (int t = 0; t < nsteps; ++t) {
    const int cur = t & 1;
    const int qa0 = qstart + t * BQ + 32 * qb;   // this wave's first query
    Step nx;
    load_step(min(t + 1, nsteps - 1), nx);

    const bool compute = kw0 < L && qa0 < L && !(CAUSAL && qa0 + 31 < kw0);
    if (compute) {
      const uint8_t* sQc = sQ0 + cur * TILE_Q;
      const uint8_t* sOc = sO0 + cur * TILE_Q;
      const bool need_mask = (qa0 + 32 > L) || (CAUSAL && qa0 < kw0 + 31);
      // S, dP: element i = query qa0 + 8(i/4) + 4g + i%4, key = key
      v16f S = v16f{}, dP = v16f{};
      {
        const uint8_t* qp = sQc + (32 * qb + n) * RS + 16 * g;
        const uint8_t* op = sOc + (32 * qb + n) * RS + 16 * g;
        const uint8_t* kp = sK + (32 * kb + n) * RS + 16 * g;
        const uint8_t* vp = sV + (32 * kb + n) * RS + 16 * g;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          S = mfma_bf16(*(const uint4*)(qp + 32 * k), *(const uint4*)(kp + 32 * k), S);
          dP = mfma_bf16(*(const uint4*)(op + 32 * k), *(const uint4*)(vp + 32 * k), dP);
        }
      }
      float p[16], ds[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 l4 = *(const float4*)&sL[cur][32 * qb + 8 * q + 4 * g];
        const float4 d4 = *(const float4*)&sD[cur][32 * qb + 8 * q + 4 * g];
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dvv[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q + e;
          float pv = __builtin_amdgcn_exp2f(fmaf(S[i], c, -lv[e]));
          if (need_mask) {
            const int qq = qa0 + 8 * q + 4 * g + e;
            const bool vis = qq < L && (!CAUSAL || qq >= key);
            pv = vis ? pv : 0.f;
          }
          p[i] = pv;
          ds[i] = pv * (dP[i] - dvv[e]);
        }
      }
      uint4 pop[2], sop[2];   // step h: queries qa0 + 16h + 8g + 0..7 of key n
      to_operands(p, pop);
      to_operands(ds, sop);
      // dV^T += dO^T P, dK^T += Q^T dS over this wave's 32 queries
#pragma unroll
      for (int dc = 0; dc < ND; ++dc)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          dv[dc] = mfma_bf16(tr_operand<RS>(sOc, 32 * qb + 16 * h2, 32 * dc, lane), pop[h2], dv[dc]);
          dk[dc] = mfma_bf16(tr_operand<RS>(sQc, 32 * qb + 16 * h2, 32 * dc, lane), sop[h2], dk[dc]);
        }
    }
    store_step(cur ^ 1, nx);
    __syncthreads();
  }

  // ---- the two waves of a key block add their partials through LDS (the tiles are free now)
  float* red = (float*)smem + (size_t)kb * (2 * ND * 16 * 64);   // [wave kb][2 ND][16][64 lanes]
  if (qb == 1) {
#pragma unroll
    for (int dc = 0; dc < ND; ++dc)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        red[((2 * dc) * 16 + e) * 64 + lane] = dk[dc][e];
        red[((2 * dc + 1) * 16 + e) * 64 + lane] = dv[dc][e];
      }
  }
  __syncthreads();
  if (qb == 1 || key >= L) return;
#pragma unroll
  for (int dc = 0; dc < ND; ++dc)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[dc][e] += red[((2 * dc) * 16 + e) * 64 + lane];
      dv[dc][e] += red[((2 * dc + 1) * 16 + e) * 64 + lane];
    }
  // lane = key, element i of chunk dc = feature 32 dc + 8(i/4) + 4g + i%4
  const long row = (long)(tok0 + key) * rowH + (long)h * D;
  const bool f32 = a.grad_f32 != 0;
#pragma unroll
  for (int dc = 0; dc < ND; ++dc)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * dc + 8 * q + 4 * g;
      store4(a.dv, row + d, f32, dv[dc][4 * q], dv[dc][4 * q + 1], dv[dc][4 * q + 2], dv[dc][4 * q + 3]);
      store4(a.dk, row + d, f32, a.sigma * dk[dc][4 * q], a.sigma * dk[dc][4 * q + 1], a.sigma * dk[dc][4 * q + 2],
             a.sigma * dk[dc][4 * q + 3]);
    }
}

// ------------------------------------------------------------------ dQ
template <int D>
struct KV16 {
  static constexpr int CH = 64 * 2 * D / 16 / 256;
  uint4 k[CH], v[CH];
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_bwd_bf16_dq_kernel(BwdArgs a) {
  constexpr int BM = 128;       // queries per workgroup (4 waves x 32)
  constexpr int BN = 64;        // keys per tile
  constexpr int NK = D / 16;
  constexpr int ND = D / 32;
  constexpr int RB = 2 * D;
  constexpr int RS = RB + 32;
  constexpr int CPR = RB / 16;
  __shared__ __attribute__((aligned(16))) uint8_t sK[2][BN * RS];
  __shared__ __attribute__((aligned(16))) uint8_t sV[2][BN * RS];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
  const int u = (j / a.nkt) * 8 + xcd;
  if (u >= a.nseq * a.H) return;
  const int qt = a.nkt - 1 - (j % a.nkt);   // longest causal query tiles first
  const int h = __builtin_amdgcn_readfirstlane(u % a.H), s = __builtin_amdgcn_readfirstlane(u / a.H);
  int tok0, L, srow0, sblk0;
  a.seq.get(s, tok0, L, srow0, sblk0);
  tok0 = __builtin_amdgcn_readfirstlane(tok0);
  L = __builtin_amdgcn_readfirstlane(L);
  const int qbase = qt * BM;
  if (qbase >= L) return;
  const int q0 = qbase + 32 * w;
  const int qi = q0 + n;
  const long rowH = (long)a.H * D;
  const uint16_t *gq = (const uint16_t*)a.q, *gk = (const uint16_t*)a.k, *gv = (const uint16_t*)a.v;
  const uint16_t* gd = (const uint16_t*)a.dout;

  auto load_tile = [&](int t, KV16<D>& st) {
    const int k0 = t * BN;
    const int rows = min(BN, L - k0);
    const long tb = (long)(tok0 + k0) * rowH + (long)h * D;
    const int nrec = ((rows - 1) * (int)rowH + D) * 2;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(gk + tb, nrec), rv = buffer_rsrc(gv + tb, nrec);
#pragma unroll
    for (int cc = 0; cc < KV16<D>::CH; ++cc) {
      const int ch = tid + cc * 256;
      const int off = (ch / CPR) * (int)rowH * 2 + (ch % CPR) * 16;
      st.k[cc] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0));
      st.v[cc] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0));
    }
  };
  auto store_tile = [&](int buf, const KV16<D>& st) {
#pragma unroll
    for (int cc = 0; cc < KV16<D>::CH; ++cc) {
      const int ch = tid + cc * 256;
      const int r = ch / CPR, cx = ch % CPR;
      *(uint4*)(&sK[buf][r * RS + cx * 16]) = st.k[cc];
      *(uint4*)(&sV[buf][r * RS + cx * 16]) = st.v[cc];
    }
  };

  // Q and dO of query qi as second operands (features 16k + 8g + 0..7); LSE, D of qi
  uint4 qa[NK], da[NK];
  float l2 = 0.f, Dq = 0.f;
  if (qi < L) {
    const long off = (long)(tok0 + qi) * rowH + (long)h * D + 8 * g;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
      qa[k] = *(const uint4*)(gq + off + 16 * k);
      da[k] = *(const uint4*)(gd + off + 16 * k);
    }
    const long li = a.seq.cu ? (long)h * a.T + tok0 + qi : ((long)s * a.H + h) * a.seq.S + qi;
    l2 = a.lse[li] * 1.44269504088896340736f;
    Dq = a.Dbuf[li];
  } else {
#pragma unroll
    for (int k = 0; k < NK; ++k) qa[k] = da[k] = make_uint4(0, 0, 0, 0);
  }

  const int kend = CAUSAL ? min(L, qbase + BM) : L;
  const int ntiles = (kend + BN - 1) / BN;
  const float c = a.c;
  v16f dq[ND];
#pragma unroll
  for (int dc = 0; dc < ND; ++dc) dq[dc] = v16f{};

  {
    KV16<D> st0;
    load_tile(0, st0);
    store_tile(0, st0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BN;
    const int cur = t & 1;
    KV16<D> nxt;
    load_tile(min(t + 1, ntiles - 1), nxt);

    const bool compute = q0 < L && !(CAUSAL && k0 > q0 + 31);
    if (compute) {
      const uint8_t* sKc = sK[cur];
      const uint8_t* sVc = sV[cur];
      const bool need_mask = (k0 + BN > L) || (CAUSAL && k0 + BN - 1 > q0);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T, dP^T: element i = key k0 + 32 kb + 8(i/4) + 4g + i%4, query qi
        v16f St = v16f{}, dPt = v16f{};
        const uint8_t* kp = sKc + (32 * kb + n) * RS + 16 * g;
        const uint8_t* vp = sVc + (32 * kb + n) * RS + 16 * g;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
          St = mfma_bf16(*(const uint4*)(kp + 32 * k), qa[k], St);
          dPt = mfma_bf16(*(const uint4*)(vp + 32 * k), da[k], dPt);
        }
        float ds[16];
        const int last = CAUSAL ? min(L - 1, qi) : L - 1;
        const int hi = last - k0 - 32 * kb - 4 * g + 1;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = __builtin_amdgcn_exp2f(fmaf(St[i], c, -l2));
          if (need_mask) pv = (8 * (i >> 2) + (i & 3) < hi) ? pv : 0.f;
          ds[i] = pv * (dPt[i] - Dq);
        }
        uint4 sop[2];   // dS^T operand: step h holds keys 32 kb + 16 h + 8g + 0..7 of query qi
        to_operands(ds, sop);
        // dQ^T += K^T dS^T: rows d = 32 dc + n, contraction over the block's 32 keys
#pragma unroll
        for (int dc = 0; dc < ND; ++dc)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2)
            dq[dc] = mfma_bf16(tr_operand<RS>(sKc, 32 * kb + 16 * h2, 32 * dc, lane), sop[h2], dq[dc]);
      }
    }
    store_tile(cur ^ 1, nxt);
    __syncthreads();
  }

  if (qi >= L) return;
  const long row = (long)(tok0 + qi) * rowH + (long)h * D;
  const bool f32 = a.grad_f32 != 0;
#pragma unroll
  for (int dc = 0; dc < ND; ++dc)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * dc + 8 * q + 4 * g;
      store4(a.dq, row + d, f32, a.sigma * dq[dc][4 * q], a.sigma * dq[dc][4 * q + 1], a.sigma * dq[dc][4 * q + 2],
             a.sigma * dq[dc][4 * q + 3]);
    }
}

hipError_t launch_attn_bwd_bf16(int D, bool causal, BwdArgs a, int max_len, hipStream_t st) {
  const long rows = (long)a.T * a.H;
  if (rows == 0) return hipSuccess;
  a.acc = nullptr;
  if (hipError_t e = launch_bwd_pre(D, false, a, st); e != hipSuccess) return e;
  const long units = (long)a.nseq * a.H;
  {
    BwdArgs b = a;
    b.nkt = (max_len + 127) / 128;
    const long grid = ((units + 7) / 8) * 8 * b.nkt;
    dim3 gd((unsigned)grid), bd(512);
    if (D == 64 && causal) attn_bwd_bf16_dkdv_kernel<64, true><<<gd, bd, 0, st>>>(b);
    else if (D == 64) attn_bwd_bf16_dkdv_kernel<64, false><<<gd, bd, 0, st>>>(b);
    else if (causal) attn_bwd_bf16_dkdv_kernel<128, true><<<gd, bd, 0, st>>>(b);
    else attn_bwd_bf16_dkdv_kernel<128, false><<<gd, bd, 0, st>>>(b);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  }
  {
    BwdArgs b = a;
    b.nkt = (max_len + 127) / 128;   // query tiles of 128
    const long grid = ((units + 7) / 8) * 8 * b.nkt;
    dim3 gd((unsigned)grid), bd(256);
    if (D == 64 && causal) attn_bwd_bf16_dq_kernel<64, true><<<gd, bd, 0, st>>>(b);
    else if (D == 64) attn_bwd_bf16_dq_kernel<64, false><<<gd, bd, 0, st>>>(b);
    else if (causal) attn_bwd_bf16_dq_kernel<128, true><<<gd, bd, 0, st>>>(b);
    else attn_bwd_bf16_dq_kernel<128, false><<<gd, bd, 0, st>>>(b);
    return hipGetLastError();
  }
}

}  // namespace mxk
