// MX GEMM with a quantizing epilogue: C = A B^T from MX payloads (MXFP8 E4M3,
// MXFP6 E2M3 / E3M2 or MXFP4 E2M1, the element formats of the block-scaled
// matrix instruction) with ROW32 (E8M0 per 32 along K) scales, fp32
// accumulation in that instruction, and C written as MXFP8 in any of ROW32 /
// COL32 / SQ32 (one pass over the fp32 tile, several scale layouts),
// optionally also in fp32.
//
// This is the "fused GEMM + Quantize" producer of "Low Precision Flash
// Attention 4: End-to-End Block-Scaled Attention for Blackwell",
// contributions paragraph (FP8 output with dual scale layouts in one pass,
// e.g. for the projections that feed the attention operands).
//
// gfx950 design:
//  * workgroup = 8 waves = one 256 x 256 tile of C, two waves per SIMD; wave w
//    holds the 128 x 64 sub-tile (rows 128 (w/4), columns 64 (w%4)) as 4 x 2
//    accumulators of v_mfma_scale_f32_32x32x64_f8f6f4, so 6 operand reads
//    from LDS feed 8 products per 64-deep step, and one wave's reads and
//    waits overlap the other's products on the SIMD;
//  * tiles in a grouped order (runs of 8 tile-rows walked column by column),
//    each XCD (blockIdx % 8) taking a contiguous run of them, so the
//    workgroups in flight on an XCD share A rows and B rows in its L2;
//  * K advances 64 per step; A and B tiles (256 rows x 8w bytes for w-bit
//    elements) go by 16-byte DMA (buffer loads with the LDS as destination)
//    into three LDS buffers, their scale pairs through registers; the DMA for
//    step k + 2 is in flight while step k is multiplied, and each step ends
//    with a wait that leaves that DMA outstanding, then a barrier;
//  * operand layout (measured): for E4M3 a lane of half g supplies bytes
//    16g..16g+15 and 32+16g..32+16g+15 of its row's 64 K values; for the 6-
//    and 4-bit formats it supplies the whole K block g (K values 32g..32g+31)
//    as a 24- or 16-byte little-endian bitstream, the packed row layout;
//  * the operands are swapped (B rows as the instruction's A operand), so a
//    lane ends with one row of C and 16 of its columns per 32 x 32 block:
//    ROW32 maxima are in-lane plus one v_permlane32_swap, COL32 maxima are
//    DPP / permlane reductions across the 32 rows of a lane half, SQ32 from
//    those; codes are regrouped with v_permlane32_swap so each lane stores 16
//    consecutive bytes of its row;
//  * encoding as in the quantizer: exact power-of-two ldexp, clamp to +-448,
//    round-to-nearest-even fp8 convert.
#include <type_traits>

#include "mx_common.h"
#include "mx_launch.h"

// waves per workgroup: one thread per scale row of the A and B tiles (256 + 256)
#define GEMM_NW 8

namespace mxk {

namespace {

MX_DEV v8i pack8g(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// max over the 32 lanes of each lane half (non-negative values; integer order = value order)
MX_DEV float half_max_nonneg(float f) {
  int v = __float_as_int(f);
  v = max(v, dpp_i32<0xB1>(v));
  v = max(v, dpp_i32<0x4E>(v));
  v = max(v, dpp_i32<0x141>(v));
  v = max(v, dpp_i32<0x140>(v));
  auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  return __int_as_float(max((int)a[0], (int)a[1]));
}

// four values times 2^sh each, clamped to +-448, packed as E4M3 codes (little-endian)
MX_DEV uint32_t enc4(float y0, float y1, float y2, float y3, int sh0, int sh1, int sh2, int sh3) {
  const float a0 = __builtin_amdgcn_fmed3f(ldexpf(y0, sh0), -448.f, 448.f);
  const float a1 = __builtin_amdgcn_fmed3f(ldexpf(y1, sh1), -448.f, 448.f);
  const float a2 = __builtin_amdgcn_fmed3f(ldexpf(y2, sh2), -448.f, 448.f);
  const float a3 = __builtin_amdgcn_fmed3f(ldexpf(y3, sh3), -448.f, 448.f);
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, r, true);
  return (uint32_t)r;
}

template <int FMT>
MX_DEV v16f mfma(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, 0, sa, 0, sb);
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled at compile time
template <int N, typename F>
MX_DEV void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// bits per element of a matrix-instruction format code (0 E4M3, 2 E2M3, 3 E3M2, 4 E2M1)
template <int FMT>
constexpr int fmt_bits() { return FMT == 0 ? 8 : FMT == 4 ? 4 : 6; }

// lane (n, g)'s operand from its row's 8w-byte K chunk in LDS; for E4M3 and E2M1 the row's 16-byte
// chunk c sits in slot c ^ sw (sw: the row's swizzle), for E2M3 / E3M2 in slot c of a padded row
template <int FMT>
MX_DEV v8i load_operand(const uint8_t* row, int g, int sw) {
  if constexpr (FMT == 0) {
    return pack8g(*(const uint4*)(row + 16 * (g ^ sw)), *(const uint4*)(row + 16 * ((2 + g) ^ sw)));
  } else if constexpr (fmt_bits<FMT>() == 6) {
    const uint2* p = (const uint2*)(row + 24 * g);
    const uint2 a = p[0], b = p[1], c = p[2];
    return v8i{(int)a.x, (int)a.y, (int)b.x, (int)b.y, (int)c.x, (int)c.y, 0, 0};
  } else {
    const uint4 a = *(const uint4*)(row + 16 * (g ^ sw));
    return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
  }
}

}  // namespace

template <int FMT>
__global__ __launch_bounds__(64 * GEMM_NW, 1) void gemm_quant_kernel(GemmArgs a) {
  // 256 x 256 tile of C: 2 x 4 waves of 128 x 64 (4 x 2 blocks, two waves per SIMD, so one
  // wave's operand reads and waits overlap the other's products).
  constexpr int NW = GEMM_NW, NTH = 64 * NW;
  constexpr int WM = 4, WN = 2;   // 32 x 32 blocks per wave along M and N
  constexpr int WCOLS = 256 / (32 * WN);        // waves along N
  constexpr int BM = 256, BN = 256;
  constexpr int W = fmt_bits<FMT>();
  constexpr int RBK = 8 * W;                        // bytes of one row per 64-deep K step
  constexpr int CPR = RBK / 16;                     // 16-byte chunks per row and step
  // E4M3 (4 chunks) and E2M1 (2 chunks): unpadded rows, chunk c of row r in slot c ^ swz(r), so the 16
  // rows one read instruction serves per pass cover all 64 banks; E2M3 / E3M2 (3 chunks, read in 8-byte
  // pieces): rows padded to 80 bytes
  constexpr bool SWZ = W != 6;
  constexpr int KST = SWZ ? RBK : RBK + 32;         // LDS row stride
  constexpr int RPS = 16 / CPR;                     // rows per 256 bytes (E4M3: 4, E2M1: 8)
  auto swz = [](int r) { return SWZ ? (r / RPS) % CPR : 0; };
  constexpr int SL = KST / 16;                      // 16-byte slots per LDS row
  constexpr int NB = BM * KST / 1024;               // 1 KB DMA blocks per tile and step
  static_assert(BM == BN && BM * KST % 1024 == 0 && 2 * NB % NW == 0, "tiles must be whole DMA blocks");
  static_assert(BM <= NTH, "one scale row per thread");
  // A and B step tiles arrive by 16-byte DMA (buffer loads straight into LDS; lane l of an
  // instruction fills bytes 16 l .. 16 l + 15 of its 1 KB block), each lane fetching the chunk its
  // slot holds: a padded row's slots past the payload hold a copy of its last chunk (never read).  One array per buffer keeps the
  // LDS reads of one buffer independent of the DMA into the other.
  __shared__ __attribute__((aligned(1024))) uint8_t sA0[BM * KST];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[BM * KST];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[BN * KST];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[BN * KST];
  __shared__ __attribute__((aligned(1024))) uint8_t sA2[BM * KST];
  __shared__ __attribute__((aligned(1024))) uint8_t sB2[BN * KST];
  __shared__ uint32_t sAs[3][BM], sBs[3][BN];   // the two scale bytes of a row for this K step

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ntiles = a.tm * a.tn;
  const int per = (ntiles + 7) / 8;
  const int tile = __builtin_amdgcn_readfirstlane((int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3));
  if (tile >= ntiles) return;
  constexpr int GM = 8;   // tile-rows per group
  const int grp = tile / (GM * a.tn), first_m = grp * GM, gm = min(a.tm - first_m, GM);
  const int in_grp = tile - grp * GM * a.tn;
  const int m0 = (first_m + in_grp % gm) * BM, n0 = (in_grp / gm) * BN;
  const int K = a.K, kb32 = K / 32;
  const int rowb = K / 8 * W;   // bytes per packed row
  const int nk = K / 64;

  // ---- staging: BM rows x 8w bytes of A and of B per step by DMA; the scale pairs in registers
  struct Stage {
    uint32_t sc;   // this thread's row's scale pair (A row tid, or B row tid - BM), or with
    int sub;       // wide scales, the step's position in the 16 bytes held in scw
  };
  static_assert(NTH == BM + BN, "one scale row per thread");
  const int rowsA = min(BM, a.M - m0), rowsB = min(BN, a.N - n0);
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(a.a + (long)m0 * rowb, rowsA * rowb);
  const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(a.b + (long)n0 * rowb, rowsB * rowb);
  const __amdgpu_buffer_rsrc_t ras = buffer_rsrc(a.as + (long)m0 * kb32, rowsA * kb32);
  const __amdgpu_buffer_rsrc_t rbs = buffer_rsrc(a.bs + (long)n0 * kb32, rowsB * kb32);
  // waves 0 .. BM/64 - 1 load A scales, the rest B scales: chosen by the scalar wave index, so the
  // resource stays in scalar registers (chosen by tid, it is per-lane to the compiler, and every
  // load through it becomes a loop over the distinct resources followed by a wait for the data)
  static_assert(BM % 64 == 0, "A and B scale rows split at a wave boundary");
  const __amdgpu_buffer_rsrc_t rsc = w < BM / 64 ? ras : rbs;
  const int srow = tid < BM ? tid : tid - BM;
  const bool wide_scales = (kb32 & 15) == 0;
  uint4 scw = make_uint4(0, 0, 0, 0);   // 8 steps of this row's scale pairs
  int kfirst = 0;                       // the first load always fetches
  // unpadded rows: block b holds rows 64 b / CPR + l / CPR, and lane l's chunk depends on l alone
  // (the swizzle of row r is (r / RPS) mod CPR = (4 b + l / 16) mod CPR), so one per-lane offset
  // serves every block, the block's part going in the scalar offset
  const int lane_off = SWZ ? (lane / CPR) * rowb + 16 * ((lane % CPR) ^ ((lane / 16) % CPR)) : 0;
  auto dma = [&](int kt, uint8_t* dA, uint8_t* dB) {
#pragma unroll
    for (int j = 0; j < 2 * NB / NW; ++j) {
      const int blk = w + NW * j;   // A blocks first, then B
      const bool isa = blk < NB;
      const int b = isa ? blk : blk - NB;
      auto* dst = (__attribute__((address_space(3))) void*)((isa ? dA : dB) + 1024 * b);
      if constexpr (SWZ) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isa ? ra : rb, dst, 16, lane_off,
                                                 __builtin_amdgcn_readfirstlane(b * (64 / CPR) * rowb + kt * RBK), 0, 0);
      } else {
        const int ch = b * 64 + lane, r = ch / SL;
        const int off = r * rowb + kt * RBK + 16 * min(ch % SL, CPR - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isa ? ra : rb, dst, 16, off, 0, 0, 0);
      }
    }
  };
  auto load = [&](int kt, Stage& st) {
    // thread t: the scale pair of A row t (t < BM) or B row t - BM.  When a row's scales are
    // 16-byte aligned (K/32 a multiple of 16) they are fetched 8 steps at a time; otherwise one
    // 16-bit load per step (K/32 is even, so a pair is 2-byte aligned).
    const int off = srow * kb32 + 2 * kt;
    if (wide_scales) {
      if ((kt & 7) == 0 || kt == kfirst) {
        scw = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsc, off - 2 * (kt & 7), 0, 0));
        kfirst = -1;
      }
      st.sub = kt & 7;   // the pair is taken from scw when stored (no wait on the load here)
    } else {
      st.sc = __builtin_amdgcn_raw_buffer_load_b16(rsc, off, 0, 0);
    }
  };
  auto store = [&](int buf, const Stage& st) {
    uint32_t sc = st.sc;
    if (wide_scales) {
      // pair `sub` of scw.  The words pass through an empty asm statement as separate values: a
      // selection among elements of one vector is folded into an indexed read, which the compiler
      // serves from a copy of the vector in memory.
      const int sub = st.sub;
      uint32_t w0 = scw.x, w1 = scw.y, w2 = scw.z, w3 = scw.w;
      asm("" : "+v"(w0), "+v"(w1), "+v"(w2), "+v"(w3));
      const uint32_t lo = (sub & 4) ? w2 : w0, hi = (sub & 4) ? w3 : w1;
      sc = (uint32_t)(((uint64_t)hi << 32 | lo) >> (16 * (sub & 3))) & 0xFFFFu;
    }
    if (tid < BM) sAs[buf][tid] = sc;
    else sBs[buf][tid - BM] = sc;
  };

  // acc[i][j]: C block (rows m0 + wr + 32 i, columns n0 + wc + 32 j); element e of
  // lane (n, g) = row + n, column + 8(e/4) + 4g + e%4
  v16f acc[WM][WN];
#pragma unroll
  for (int i = 0; i < WM; ++i)
#pragma unroll
    for (int j = 0; j < WN; ++j) acc[i][j] = v16f{};
  const int wr = 32 * WM * (w / WCOLS), wc = 32 * WN * (w % WCOLS);
  int sa_prev[WM], sb_prev[WN];   // scale operands of the last products, pinned
#pragma unroll
  for (int i = 0; i < WM; ++i) sa_prev[i] = 0;
#pragma unroll
  for (int j = 0; j < WN; ++j) sb_prev[j] = 0;

  // the three step buffers, each its own array (named by a constant at every use, so the LDS reads
  // of one buffer carry no dependence on the DMA into another)
  auto bufA = [&](int c) -> uint8_t* { return c == 0 ? sA0 : (c == 1 ? sA1 : sA2); };
  auto bufB = [&](int c) -> uint8_t* { return c == 0 ? sB0 : (c == 1 ? sB1 : sB2); };
  // one 64-deep step from LDS buffer cur: operands, then the WM x WN products
  auto compute = [&](const int cur) __attribute__((always_inline)) {
    v8i ao[WM], bo[WN];
    int sa[WM], sb[WN];
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      ao[i] = load_operand<FMT>(bufA(cur) + (wr + 32 * i + n) * KST, g, swz(n));
      sa[i] = (int)(sAs[cur][wr + 32 * i + n] >> (8 * g));
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      bo[j] = load_operand<FMT>(bufB(cur) + (wc + 32 * j + n) * KST, g, swz(n));
      sb[j] = (int)(sBs[cur][wc + 32 * j + n] >> (8 * g));
    }
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
      for (int j = 0; j < WN; ++j) acc[i][j] = mfma<FMT>(bo[j], ao[i], acc[i][j], sb[j], sa[i]);
#pragma unroll
    for (int i = 0; i < WM; ++i) {
      keep(sa_prev[i]);
      sa_prev[i] = sa[i];
    }
#pragma unroll
    for (int j = 0; j < WN; ++j) {
      keep(sb_prev[j]);
      sb_prev[j] = sb[j];
    }
  };
  // Three buffers, two steps of DMA in flight: step kt computes from buffer kt % 3 while the DMA for
  // step kt + 2 fills buffer (kt + 2) % 3 (read last in step kt - 1, before the barrier that ended
  // it).  A step ends with a wait for everything but its own DMA (so the DMA for step kt + 1 and
  // the scale loads have landed, and its LDS accesses are done) and a barrier; a __syncthreads()
  // there would also wait for this step's DMA, one step of prefetch only (measured: 30% of the
  // kernel's time is then DMA latency).
  constexpr int NDMA = 2 * NB / NW;   // DMA instructions per wave and step
  static_assert(NDMA < 64, "vmcnt field");
  auto end_step = [&](bool dma_in_flight) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);   // no LDS access moves across the barrier
    // s_waitcnt: vmcnt bits 3:0 and 15:14, expcnt 6:4 (not waited), lgkmcnt 11:8 (0)
    if (dma_in_flight) __builtin_amdgcn_s_waitcnt((NDMA & 15) | ((NDMA >> 4) << 14) | (7 << 4));
    else __builtin_amdgcn_s_waitcnt(7 << 4);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  };
  {
    Stage s0, s1;
    load(0, s0);
    dma(0, sA0, sB0);
    if (nk > 1) {
      load(1, s1);
      dma(1, sA1, sB1);
    }
    store(0, s0);
    if (nk > 1) store(1, s1);
  }
  __syncthreads();
  auto step = [&](int kt, auto cur_c) __attribute__((always_inline)) {
    constexpr int CUR = decltype(cur_c)::value, NXT = (CUR + 2) % 3;
    const bool ahead = kt + 2 < nk;
    Stage s2;
    if (ahead) {
      load(kt + 2, s2);
      dma(kt + 2, bufA(NXT), bufB(NXT));
    }
    compute(CUR);
    if (ahead) store(NXT, s2);
    end_step(ahead);
  };
  int kt = 0;
  for (; kt + 2 < nk; kt += 3) {
    step(kt, std::integral_constant<int, 0>{});
    step(kt + 1, std::integral_constant<int, 1>{});
    step(kt + 2, std::integral_constant<int, 2>{});
  }
  if (kt < nk) step(kt, std::integral_constant<int, 0>{});
  if (kt + 1 < nk) step(kt + 1, std::integral_constant<int, 1>{});
  keep(acc[WM - 1][WN - 1][0]);
#pragma unroll
  for (int i = 0; i < WM; ++i) keep(sa_prev[i]);
#pragma unroll
  for (int j = 0; j < WN; ++j) keep(sb_prev[j]);

  // ---- epilogue, per 32 x 32 block
  const long ldc = a.N;
  // one 32 x 32 block (i, j); every call site indexes acc with constants, so the accumulators
  // stay in registers (a loop over dynamic indices would put the array in scratch memory)
  auto block = [&](const v16f& c, const int i, const int j) __attribute__((always_inline)) {
      const int row = m0 + wr + 32 * i + n;      // this lane's row
      const int col0 = n0 + wc + 32 * j;         // first column of the block
      const bool row_ok = row < a.M;
      // fp32 copy: dword group q holds columns col0 + 8q + 4g + 0..3
      if (a.c32 && row_ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cc = col0 + 8 * q + 4 * g;
          float* dst = a.c32 + (long)row * ldc + cc;
          if (cc + 3 < a.N) {
            *(float4*)dst = make_float4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3]);
          } else {
            for (int e = 0; e < 4; ++e)
              if (cc + e < a.N) dst[e] = c[4 * q + e];
          }
        }
      }
      // maxima: per row (ROW32), per column (COL32), per block (SQ32)
      float rm = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) rm = fmaxf(rm, fabsf(c[e]));
      rm = half_swap_max(rm);                    // the row's 32 columns
      float cm[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) cm[e] = half_max_nonneg(fabsf(c[e]));   // the column's 32 rows
      float bmx = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) bmx = fmaxf(bmx, cm[e]);
      bmx = half_swap_max(bmx);
      // encode one layout: per-element shifts, then regroup so lane half g holds columns 16g + 0..15
      auto emit = [&](uint8_t* data, const int* sh) {
        uint32_t dw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          dw[q] = enc4(c[4 * q], c[4 * q + 1], c[4 * q + 2], c[4 * q + 3], sh[4 * q], sh[4 * q + 1], sh[4 * q + 2],
                       sh[4 * q + 3]);
        auto s02 = __builtin_amdgcn_permlane32_swap(dw[0], dw[2], false, false);
        auto s13 = __builtin_amdgcn_permlane32_swap(dw[1], dw[3], false, false);
        const int cs = col0 + 16 * g;
        if (row_ok) {
          uint8_t* dst = data + (long)row * ldc + cs;
          const uint32_t v[4] = {s02[0], s02[1], s13[0], s13[1]};
          if (cs + 15 < a.N) {
            *(uint4*)dst = make_uint4(v[0], v[1], v[2], v[3]);
          } else {
            for (int b = 0; b < 16 && cs + b < a.N; ++b) dst[b] = (uint8_t)(v[b >> 2] >> (8 * (b & 3)));
          }
        }
      };
      const int nbn = (a.N + 31) / 32;
      if (a.layouts & 1) {   // ROW32: one scale per row and 32 columns
        const int k = scale_code(rm);
        int sh[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sh[e] = 127 - k;
        emit(a.row_data, sh);
        if (g == 0 && row_ok && col0 < a.N) a.row_scale[(long)row * nbn + col0 / 32] = (uint8_t)k;
      }
      if (a.layouts & 2) {   // COL32: one scale per column and 32 rows
        int sh[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sh[e] = 127 - scale_code(cm[e]);
        emit(a.col_data, sh);
        if (n == 0 && m0 + wr + 32 * i < a.M) {   // blocks wholly past the last row have no scales
          const int rb = (m0 + wr + 32 * i) / 32;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int cc = col0 + 8 * (e >> 2) + 4 * g + (e & 3);
            if (cc < a.N) a.col_scale[(long)rb * ldc + cc] = (uint8_t)(127 - sh[e]);
          }
        }
      }
      if (a.layouts & 4) {   // SQ32: one scale per 32 x 32 block
        const int k = scale_code(bmx);
        int sh[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) sh[e] = 127 - k;
        emit(a.sq_data, sh);
        if (lane == 0 && m0 + wr + 32 * i < a.M && col0 < a.N)
          a.sq_scale[(long)((m0 + wr + 32 * i) / 32) * nbn + col0 / 32] = (uint8_t)k;
      }
  };
  static_for<WM>([&](auto I) { static_for<WN>([&](auto J) { block(acc[I][J], I, J); }); });
}

hipError_t launch_gemm_quantize(GemmArgs a, hipStream_t st) {
  constexpr int TILE = 256;
  a.tm = (a.M + TILE - 1) / TILE;
  a.tn = (a.N + TILE - 1) / TILE;
  const long ntiles = (long)a.tm * a.tn;
  if (ntiles == 0) return hipSuccess;
  const long grid = (ntiles + 7) / 8 * 8;
  dim3 g((unsigned)grid), b(64 * GEMM_NW);
  switch (a.fmt) {
    case 0: gemm_quant_kernel<0><<<g, b, 0, st>>>(a); break;
    case 2: gemm_quant_kernel<2><<<g, b, 0, st>>>(a); break;
    case 3: gemm_quant_kernel<3><<<g, b, 0, st>>>(a); break;
    case 4: gemm_quant_kernel<4><<<g, b, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mxk
