// Fused MXFP8 attention forward for gfx950.
//
// What is computed follows "Low-Precision FlashAttention-4: End-to-End
// Block-Scaled Attention for NVIDIA Blackwell", sections "1. End-to-End
// Block-Scaled GEMM Fusion" (S = Q K^T and P V on block-scaled operands, no
// HBM round trip in between) and "2. Synchronized Online Softmax with Dynamic
// Scaling" (FP32 running max and sum), and "Low Precision Flash Attention 4:
// End-to-End Block-Scaled Attention for Blackwell", forward/backward
// paragraph (the FP32 softmax result is converted to MXFP8, its block scales
// taken from the maximum the softmax already holds).
//
// gfx950 design (not the pages' Blackwell design):
//  * Each wavefront owns 32 queries and computes S^T = K Q^T with
//    v_mfma_scale_f32_32x32x64_f8f6f4, so every lane holds one query and 16
//    keys of each 32-key block: the row max needs one cross-lane step and the
//    block scale of P is set per lane.
//  * Softmax runs in the log2 domain under an integer frame M (moved lazily,
//    once ceil(max t) exceeds it by more than 8), so rescaling O and l is an
//    exact power of two and P's codes do not depend on how keys are tiled
//    (up to the fp32 rounding of the argument t - M).
//  * P's block amax is 2^(block max of t - M), so its E8M0 scale follows
//    from the maxima already reduced for M, with no extra exp (and no
//    dependence on the accuracy of the hardware exp2).  The fp32->fp8 convert
//    (which divides by the E8M0 scale) saturates through the wave's MODE
//    setting, so no clamp precedes it.
//  * The K rows of each 32-key block sit in LDS in an order that makes each
//    lane half's 16 elements of S^T 16 consecutive keys, the order in which
//    the P V product takes P (no lane-half exchange of P); V^T comes from a
//    row-major LDS tile through ds_read_b64_tr_b8, in that key order.
//  * K and V tiles of 64 or 128 keys go from HBM straight into LDS (16-byte
//    buffer loads with the LDS as destination, no staging registers), into
//    rows whose 16-byte chunks are XOR-swizzled by row so the operand reads
//    spread over the banks; two LDS buffers, the next tile's loads in flight
//    while the current one is computed, one barrier per tile, and three (or
//    two) workgroups per CU so one's softmax overlaps another's MFMAs.  Workgroups are ordered so that each XCD works
//    through whole heads, longest (causal) query tiles first, keeping a
//    head's K/V in that XCD's L2.
#include "mx_common.h"
#include "mx_launch.h"

namespace mxk {

template <int OA, int OB, int FMT = 0>
MX_DEV v16f mfma32(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT, FMT, OA, sa, OB, sb);
}

MX_DEV v8i pack8(uint4 lo, uint4 hi) {
  v8i r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

// Bits per element of the Q / K payload: E4M3 (code 0), E2M3 / E3M2 (2, 3), E2M1 (4).
template <int QF>
constexpr int qk_bits() { return QF == 0 ? 8 : QF == 4 ? 4 : 6; }

// Operand of one QK^T product (64 contraction indices = 32-element blocks 2c, 2c + 1) for lane half
// g, from a packed Q or K row.  E4M3: bytes 16g..16g+15 and 32+16g..32+16g+15 of the chunk.  MXFP6 /
// MXFP4: the whole block 2c + g as the instruction's little-endian bitstream (24 or 16 bytes in the
// first dwords; measured layout of the scaled instruction's format fields).
template <int QF>
MX_DEV v8i qk_operand(const uint8_t* row, int c, int g) {
  if constexpr (QF == 0) {
    return pack8(*(const uint4*)(row + 64 * c + 16 * g), *(const uint4*)(row + 64 * c + 32 + 16 * g));
  } else if constexpr (qk_bits<QF>() == 6) {
    const uint2* p = (const uint2*)(row + 24 * (2 * c + g));
    const uint2 x = p[0], y = p[1], z = p[2];
    return v8i{(int)x.x, (int)x.y, (int)y.x, (int)y.y, (int)z.x, (int)z.y, 0, 0};
  } else {
    const uint4 x = *(const uint4*)(row + 16 * (2 * c + g));
    return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  }
}

// Operand of one QK^T product read from a K tile in LDS at precomputed lane byte offsets (o0: the
// first chunk or the whole operand, o1: the second E4M3 chunk).
template <int QF>
MX_DEV v8i qk_operand_at(const uint8_t* tile, int o0, int o1) {
  if constexpr (QF == 0) {
    return pack8(*(const uint4*)(tile + o0), *(const uint4*)(tile + o1));
  } else if constexpr (qk_bits<QF>() == 6) {
    const uint2* p = (const uint2*)(tile + o0);
    const uint2 x = p[0], y = p[1], z = p[2];
    return v8i{(int)x.x, (int)x.y, (int)y.x, (int)y.y, (int)z.x, (int)z.y, 0, 0};
  } else {
    const uint4 v = *(const uint4*)(tile + o0);
    return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
  }
}

MX_DEV v2i lds_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((v2i __attribute__((address_space(3)))*)(p));
}

// Key tile and workgroups per CU: 64-key tiles at three workgroups (three waves per SIMD, at most
// 168 VGPRs) wherever the variant fits that without spilling, for the extra wave that hides the
// softmax's latencies (E4M3 causal: 3.11 -> 3.01-3.05 ms, E2M1 -6%); else 128-key tiles at two
// (the E4M3 variants other than causal with bf16 output spill one or two registers at 168).
template <int D, bool CAUSAL, bool OUT_BF16, int QF>
constexpr bool fwd_three_waves() {
  return D == 64 || QF != 0 || (CAUSAL && OUT_BF16);
}

template <int D, int NW, bool CAUSAL, bool OUT_BF16, int QF>
__global__ __launch_bounds__(NW * 64, (fwd_three_waves<D, CAUSAL, OUT_BF16, QF>() ? 3 : 2)) void attn_fwd_kernel(FwdArgs a) {
  constexpr int BM = 32 * NW;   // queries per workgroup
  constexpr int BN = fwd_three_waves<D, CAUSAL, OUT_BF16, QF>() ? 64 : 128;   // keys per tile
  constexpr int KB = BN / 32;   // 32-key blocks per tile
  static_assert(KB % 2 == 0, "block maxima are exchanged in pairs of blocks");
  constexpr int KH = BN / 64;   // 64-key halves per tile (one P V contraction each)
  constexpr int NC = D / 64;    // 64-feature chunks of the QK^T contraction
  constexpr int ND = D / 32;    // 32-feature chunks of O
  constexpr int KRB = D * qk_bits<QF>() / 8;   // payload bytes of one Q or K row
  // K and V tiles arrive by 16-byte DMA (buffer loads straight into LDS, no staging registers).
  // Rows of a power-of-two number of 16-byte chunks are stored unpadded, chunk j of a row in a
  // slot XOR-swizzled by the row, so the operand reads spread over the banks: K, read a row per
  // lane (16-byte reads, 16 lanes a pass), swizzles by (r / rows per 256 bytes) mod chunks, which
  // gives the 16 rows of a pass 16 distinct bank groups; V, read by 8-byte transpose reads, by
  // r mod chunks (measured conflict-free for both; K swizzled by r mod chunks instead took 1.75x
  // (128-byte rows) and 3.3x (64-byte rows) the time per read).  MXFP6 K rows (3 or 6 chunks) get
  // one spare slot instead (a copy of the last chunk, never read), which staggers the rows across
  // the banks.
  constexpr int CPRV = D / 16;                        // chunks per V row
  constexpr int CPRK = KRB / 16;                      // chunks of payload per K row
  constexpr bool KPOW2 = (CPRK & (CPRK - 1)) == 0;
  constexpr int SLK = KPOW2 ? CPRK : CPRK + 1;        // K row slots (MXFP6: one spare slot)
  constexpr int KRS = 16 * SLK;                       // LDS row stride of the K tile
  constexpr int SWZV = CPRV - 1, SWZK = KPOW2 ? SLK - 1 : 0;
  constexpr int RPWK = KRS >= 256 ? 1 : 256 / KRS;     // K rows per 256 bytes (one pass of the banks)
  auto swzk = [](int r) { return (r / RPWK) & SWZK; };
  // K rows of each 32-key block are stored in the order that makes the S^T product's output element
  // i of lane half g key 16 g + i of the block: LDS row p (= output row 8(i/4) + 4g + i%4) holds key
  // korder(p).  P then comes out of the softmax with each lane half holding its 16 consecutive keys,
  // the order the P V product takes them in, with no lane-half exchange.
  auto korder = [](int p) { return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3); };
  constexpr int NBK = BN * KRS / 1024, NBV = BN * D / 1024;   // 1 KB DMA blocks (one wave instruction each)
  static_assert(BN * KRS % 1024 == 0 && BN * D % 1024 == 0, "tiles must be whole DMA blocks");
  constexpr float kLazy = 8.f;  // largest log2 of p before the frame moves
  constexpr int NT = NW * 64;
  static_assert(BN * D / 16 % NT == 0, "tile chunks must divide among the threads");
  // two buffers: the tile being computed and the next one, written while it is computed
  // one array per buffer: the LDS reads of one buffer stay independent of the DMA into the other
  __shared__ __attribute__((aligned(1024))) uint8_t sK0[BN * KRS];
  __shared__ __attribute__((aligned(1024))) uint8_t sK1[BN * KRS];
  __shared__ __attribute__((aligned(1024))) uint8_t sV0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint8_t sV1[BN * D];
  // The tile's E8M0 scales arrive by DMA too, one 4-byte LDS word per lane: K's ROW32 scale word of
  // each key; V's COL32 scale bytes (zero-extended by the byte-sized DMA) as [dc][64 hh + l] = the
  // scale of (key block 2 hh + l / 32, d = 32 dc + l % 32).  One array per buffer, so the reads of one
  // carry no dependence on the DMA into the other.
  __shared__ uint32_t sKs0[BN], sKs1[BN];
  __shared__ uint32_t sVs0[ND][BN], sVs1[ND][BN];

  saturating_fp8_converts();
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform

  // ---- work decode: XCD x = id % 8 takes (sequence, head) units x, x+8, ...;
  // within a unit, the longest query tile first.
  const int id = blockIdx.x, xcd = id & 7, j = id >> 3;
  const int u = (j / a.nqt) * 8 + xcd;
  if (u >= a.nseq * a.H) return;
  const int qt = a.nqt - 1 - (j % a.nqt);
  const int h = __builtin_amdgcn_readfirstlane(u % a.H), s = __builtin_amdgcn_readfirstlane(u / a.H);
  int tok0, L, srow0, sblk0;
  a.seq.get(s, tok0, L, srow0, sblk0);
  // wave-uniform (they come from the workgroup index): lets the buffer resources live in SGPRs
  tok0 = __builtin_amdgcn_readfirstlane(tok0);
  L = __builtin_amdgcn_readfirstlane(L);
  srow0 = __builtin_amdgcn_readfirstlane(srow0);
  sblk0 = __builtin_amdgcn_readfirstlane(sblk0);
  const int qbase = qt * BM;
  if (qbase >= L) return;
  const int q0 = qbase + 32 * w;
  const int qi = q0 + n;
  const long rowH = (long)a.H * D;       // V and O row stride
  const long rowHk = (long)a.H * KRB;    // Q and K payload row stride

  // ---- staging of one K/V tile: payload and scales by buffer loads whose destination is the LDS.
  // Each tile gets scalar buffer resources that end with the sequence, so rows
  // (and scale blocks) past its end read as zero: no clamps, no branches, and no
  // staging registers.  (Through registers, the scales cost 4.5% of the kernel's time and five
  // registers held across the tile; a byte-sized load into LDS writes its byte zero-extended to a
  // 4-byte word per lane, measured, so the V scales land one per word.)
  const int KSB = D / 32;   // bytes per K ROW32 scale word
  // lane l of a DMA instruction fills bytes 16 l .. 16 l + 15 of its 1 KB block (measured)
  const int kend = CAUSAL ? min(L, qbase + BM) : L;   // keys this workgroup visits
  const int ntiles = (kend + BN - 1) / BN;
  // The next tile to load: its index and wave-uniform pointers to its K, V rows and scales of this
  // head, advanced by one tile per load with 64-bit scalar adds (a product of tile index and row
  // stride per load would be computed on the vector unit and moved back to scalar registers).
  // Tiles load in order 0, 1, ..., the last one possibly twice.
  struct NextTile {
    const uint8_t *k, *v, *ks, *vs;
    int t;
  };
  NextTile nt{a.k + (long)tok0 * rowHk + (long)h * KRB, a.v + (long)tok0 * rowH + (long)h * D,
              a.ks + ((long)srow0 * a.H + h) * KSB, a.vs + ((long)sblk0 * a.H + h) * D, 0};
  const long kstep = (long)BN * rowHk, vstep = (long)BN * rowH;
  const long ksstep = (long)BN * a.H * KSB, vsstep = (long)KB * a.H * D;
  auto advance = [&]() {
    if (nt.t + 1 < ntiles) {
      ++nt.t;
      nt.k += kstep;
      nt.v += vstep;
      nt.ks += ksstep;
      nt.vs += vsstep;
    }
  };
  auto dma_tile = [&](uint8_t* dK, uint8_t* dV) {
    const int rows = min(BN, L - nt.t * BN);   // >= 1
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(nt.k, (rows - 1) * (int)rowHk + KRB);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(nt.v, (rows - 1) * (int)rowH + D);
#pragma unroll
    for (int j = 0; j < (NBK + NW - 1) / NW; ++j) {
      const int blk = w + NW * j;
      if (NBK % NW == 0 || blk < NBK) {
        const int ch = blk * 64 + lane, r = ch / SLK;
        const int lc = (ch % SLK) ^ swzk(r);      // chunk this slot holds
        const int off = korder(r) * (int)rowHk + 16 * min(lc, CPRK - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (__attribute__((address_space(3))) void*)(dK + 1024 * blk), 16,
                                                 off, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < NBV / NW; ++j) {
      const int blk = w + NW * j;
      const int ch = blk * 64 + lane, r = ch / CPRV;
      const int off = r * (int)rowH + 16 * ((ch % CPRV) ^ (r & SWZV));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(dV + 1024 * blk), 16,
                                               off, 0, 0, 0);
    }
  };
  // the tile's scales by DMA: per 64-key half one dword (K) and ND byte (V) instructions, spread
  // over the waves
  auto dma_scales = [&](uint32_t* dKs, uint32_t (*dVs)[BN]) {
    const int rows = min(BN, L - nt.t * BN);
    const __amdgpu_buffer_rsrc_t rks = buffer_rsrc(nt.ks, (rows - 1) * a.H * KSB + KSB);
    const int nblk = (rows + 31) / 32;
    const __amdgpu_buffer_rsrc_t rvs = buffer_rsrc(nt.vs, (nblk - 1) * a.H * D + D);
#pragma unroll
    for (int hh = 0; hh < KH; ++hh) {
      const int kk = 64 * hh + lane;   // key of this lane in the tile
#pragma unroll
      for (int j = 0; j <= ND; ++j) {
        if (((1 + ND) * hh + j) % NW != w) continue;
        if (j == 0) {
          auto* dst = (__attribute__((address_space(3))) void*)(dKs + 64 * hh);
          if constexpr (D == 128) __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, dst, 4, kk * a.H * KSB, 0, 0, 0);
          else __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, dst, 2, kk * a.H * KSB, 0, 0, 0);
        } else {
          const int dc = j - 1;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rvs, (__attribute__((address_space(3))) void*)(dVs[dc] + 64 * hh),
                                                   1, (kk >> 5) * a.H * D + (kk & 31) + 32 * dc, 0, 0, 0);
        }
      }
    }
  };

  // lane byte offsets of the QK operand chunks in a K tile (row n of key block 0): key block kb adds
  // 32 kb rows, a whole number of swizzle periods, so its chunks sit at a constant distance.  An
  // empty asm statement hides their arithmetic, so each tile's reads use these four registers plus
  // constant offsets (otherwise every read's full address is kept or recomputed).
  static_assert(32 % (RPWK * (SWZK + 1)) == 0, "key blocks span whole swizzle periods");
  int kofs[NC][2];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int x = swzk(n);
    if constexpr (QF == 0) {
      kofs[c][0] = n * KRS + 16 * ((4 * c + g) ^ x);
      kofs[c][1] = n * KRS + 16 * ((4 * c + 2 + g) ^ x);
      asm("" : "+v"(kofs[c][0]), "+v"(kofs[c][1]));
    } else if constexpr (qk_bits<QF>() == 6) {
      kofs[c][0] = n * KRS + 24 * (2 * c + g);
      kofs[c][1] = 0;
      asm("" : "+v"(kofs[c][0]));
    } else {
      kofs[c][0] = n * KRS + 16 * ((2 * c + g) ^ x);
      kofs[c][1] = 0;
      asm("" : "+v"(kofs[c][0]));
    }
  }

  // ---- Q as the B operand (resident for the whole key loop)
  v8i qa[NC];
  uint32_t qsc = 0;
  if (qi < L) {
    const uint8_t* qp = a.q + (long)(tok0 + qi) * rowHk + (long)h * KRB;
#pragma unroll
    for (int c = 0; c < NC; ++c) qa[c] = qk_operand<QF>(qp, c, g);
    const long srow = ((long)(srow0 + qi) * a.H + h);
    uint32_t wq = (D == 128) ? *(const uint32_t*)(a.qs + srow * 4) : *(const uint16_t*)(a.qs + srow * 2);
    qsc = wq >> (8 * g);
  } else {
#pragma unroll
    for (int c = 0; c < NC; ++c) qa[c] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  }


  v16f o[ND];
#pragma unroll
  for (int dc = 0; dc < ND; ++dc) o[dc] = v16f{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.c;
  uint32_t vsc_prev[KH];   // scale operands of the last P V products, pinned until they finish
  int psc_prev[KH];
#pragma unroll
  for (int hh = 0; hh < KH; ++hh) vsc_prev[hh] = psc_prev[hh] = 0;

  // one tile's products and softmax from LDS buffer cur; hook() (the next tile's scale loads and DMA) runs right after
  // the S products are issued, or at once on a wave with nothing to compute: a wave's DMA issue can
  // wait on the CU's memory pipe, and its S products then already run (measured -3% against issuing
  // it before them)
  auto tile_body = [&](const int t, const int cur, auto&& hook) __attribute__((always_inline)) {
    const int k0 = t * BN;

    const bool compute = q0 < L && !(CAUSAL && k0 > q0 + 31);   // skip tiles above this wave's diagonal
    if (compute) {
      const uint8_t* sKc = cur ? sK1 : sK0;
      const uint8_t* sVc = cur ? sV1 : sV0;
      const uint32_t* sKsc = cur ? sKs1 : sKs0;
      const uint32_t (*sVsc)[BN] = cur ? sVs1 : sVs0;
      // ---- S^T = K Q^T : st[kb] element i holds key k0 + 32 kb + 16g + i (K rows in korder), query qi
      v16f st[KB];
      uint32_t ksc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        const uint8_t* kt = sKc + kb * 32 * KRS;
        ksc[kb] = sKsc[kb * 32 + korder(n)] >> (8 * g);
        v16f acc = v16f{};
        acc = mfma32<0, 0, QF>(qk_operand_at<QF>(kt, kofs[0][0], kofs[0][1]), qa[0], acc, ksc[kb], qsc);
        if constexpr (NC > 1)
          acc = mfma32<2, 2, QF>(qk_operand_at<QF>(kt, kofs[NC - 1][0], kofs[NC - 1][1]), qa[NC - 1], acc, ksc[kb], qsc);
        st[kb] = acc;
      }
      hook();
      const bool need_mask = (k0 + BN > L) || (CAUSAL && k0 + BN - 1 > q0);
      if (need_mask) {
        // element i is key k0 + 32 kb + 16 g + i: visible iff i < hi
        const int last = CAUSAL ? min(L - 1, qi) : L - 1;   // last visible key of this query
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const int hi = last - k0 - 32 * kb - 16 * g + 1;
#pragma unroll
          for (int i = 0; i < 16; ++i) st[kb][i] = (i < hi) ? st[kb][i] : -INFINITY;
        }
      }
      // ---- block maxima, frame update
      // per lane the max of its 16 keys of each block; then blocks in pairs: one half swap gives
      // lanes 0-31 both halves of block 2j and lanes 32-63 both halves of block 2j + 1, a second
      // (of the pairwise maximum with itself) hands each lane both blocks' maxima
      float bm[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        float m = st[kb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) m = fmaxf(m, st[kb][i]);
        bm[kb] = m;
      }
#pragma unroll
      for (int kb = 0; kb < KB; kb += 2) {
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(bm[kb]), __float_as_uint(bm[kb + 1]), false, false);
        const float x = fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
        const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        bm[kb] = __uint_as_float(b[0]);
        bm[kb + 1] = __uint_as_float(b[1]);
      }
      // S has been read: this tile's S products and the previous tile's P V products are done
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) keep(ksc[kb]);
#pragma unroll
      for (int hh = 0; hh < KH; ++hh) {
        keep(vsc_prev[hh]);
        keep(psc_prev[hh]);
      }
      // Lazy frame: M moves (and O, l are rescaled by 2^(M_old - M_new)) only once the tile's
      // ceil(max) exceeds it by more than kLazy, so p stays below 2^kLazy.  In exact arithmetic
      // every frame gives P^ the same codes (its scales absorb the power of two) and the same
      // O and LSE; in fp32 the argument S c - M rounds at the frame's magnitude.
      float tmax = bm[0];
#pragma unroll
      for (int kb = 1; kb < KB; ++kb) tmax = fmaxf(tmax, bm[kb]);
      const float m_tile = ceilf(tmax * c);
      if (m_tile > m_run + kLazy) {
        const float alpha = (m_run == -INFINITY) ? 0.f : ldexpf(1.f, (int)(m_run - m_tile));
#pragma unroll
        for (int dc = 0; dc < ND; ++dc) o[dc] *= alpha;
        l_run *= alpha;
        m_run = m_tile;
      }
      const float negM = -m_run;
      // ---- p = 2^(S c - M), running sum
      // four partial sums: independent add chains (one chain held every p live until its add,
      // which pushed the kernel past its register budget)
      float ps[4];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(fmaf(st[kb][i], c, negM));
          st[kb][i] = p;
          if (kb == 0 && i < 4) ps[i] = p;   // (0 + p would cost an add: -0 + 0 is +0)
          else ps[i & 3] += p;
        }
      l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
      int kc[KB];
      float sc[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // block amax of p is 2^(block max of t - M): its scale straight from that exponent
        kc[kb] = exp2_scale_code(fmaf(bm[kb], c, negM));
        sc[kb] = e8m0_f32(kc[kb]);
      }
      // ---- P -> E4M3 codes: dword q of block kb holds keys 16g + 4q + 0..3
      uint32_t dw[KB][4];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          dw[kb][q] = cvt4_scaled_fp8(st[kb][4 * q], st[kb][4 * q + 1], st[kb][4 * q + 2], st[kb][4 * q + 3], sc[kb]);
        }
      // ---- per 64-key half hh: lane half g holds keys 16g + 0..15 of each of its two blocks, in
      // order (the K row order above); O^T += V^T P^T (V^T rows d = 32 dc + lane%32, through LDS
      // transpose reads)
      const int G = lane >> 4, i16 = lane & 15;
      const int rowofs = 16 * (G >> 1) + (i16 >> 1);
#pragma unroll
      for (int hh = 0; hh < KH; ++hh) {
        v8i pb;
#pragma unroll
        for (int b2 = 0; b2 < 2; ++b2)
#pragma unroll
          for (int q = 0; q < 4; ++q) pb[4 * b2 + q] = dw[2 * hh + b2][q];
        const int psc = g ? kc[2 * hh + 1] : kc[2 * hh];
        uint32_t vsc = 0;
#pragma unroll
        for (int dc = 0; dc < ND; ++dc) vsc |= sVsc[dc][64 * hh + lane] << (8 * dc);
#pragma unroll
        for (int dc = 0; dc < ND; ++dc) {
          // rows vrow, +8, +32, +40 share vrow's swizzle; chunk 2 dc + (G & 1), half i16 & 1
          const int vrow = 64 * hh + rowofs;
          const uint8_t* vp = sVc + vrow * D + 16 * ((2 * dc + (G & 1)) ^ (vrow & SWZV)) + 8 * (i16 & 1);
          v2i r0 = lds_tr8(vp), r1 = lds_tr8(vp + 8 * D), r2 = lds_tr8(vp + 32 * D), r3 = lds_tr8(vp + 40 * D);
          v8i va = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
          if (dc == 0) o[0] = mfma32<0, 0>(va, pb, o[0], vsc, psc);
          if (dc == 1) o[1] = mfma32<1, 0>(va, pb, o[1], vsc, psc);
          if constexpr (ND > 2) {
            if (dc == 2) o[2] = mfma32<2, 0>(va, pb, o[2], vsc, psc);
            if (dc == 3) o[3] = mfma32<3, 0>(va, pb, o[3], vsc, psc);
          }
        }
        vsc_prev[hh] = vsc;
        psc_prev[hh] = psc;
      }
    } else {
      hook();
    }
  };
  dma_scales(sKs0, sVs0);
  dma_tile(sK0, sV0);
  advance();
  __syncthreads();
  // the next tile's DMA and scale loads are in flight while this one is computed (past the last
  // tile the last one is fetched again into the free buffer, which keeps the loop free of branches
  // around them); two tiles per iteration so each buffer is named at compile time
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    tile_body(t, 0, [&]() { dma_scales(sKs1, sVs1); dma_tile(sK1, sV1); });
    advance();
    __syncthreads();
    tile_body(t + 1, 1, [&]() { dma_scales(sKs0, sVs0); dma_tile(sK0, sV0); });
    advance();
    __syncthreads();
  }
  if (t < ntiles) tile_body(t, 0, [&]() {});

  // ---- epilogue: O = O^T / l, LSE = ln2 (M + log2 l).  Each lane half summed
  // p over its 16 keys of every block: the row sum adds both halves.
  l_run += __shfl_xor(l_run, 32, 64);
  keep(o[ND - 1][0]);
#pragma unroll
  for (int hh = 0; hh < KH; ++hh) {
    keep(vsc_prev[hh]);
    keep(psc_prev[hh]);
  }
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

hipError_t launch_attn_fwd(int D, bool causal, bool out_bf16, int qk_fmt, FwdArgs a, int max_len, hipStream_t st) {
  constexpr int NW = 4;
  a.nqt = (max_len + 32 * NW - 1) / (32 * NW);
  const long units = (long)a.nseq * a.H;
  const long grid = ((units + 7) / 8) * 8 * a.nqt;
  if (grid == 0) return hipSuccess;
  dim3 g((unsigned)grid), b(NW * 64);
#define MX_FWD_CASE(DD, CC, OB, QF)                                            \
  if (D == DD && causal == CC && out_bf16 == OB && qk_fmt == QF) {              \
    attn_fwd_kernel<DD, NW, CC, OB, QF><<<g, b, 0, st>>>(a);                    \
    return hipGetLastError();                                                   \
  }
#define MX_FWD_FMTS(DD, CC, OB) \
  MX_FWD_CASE(DD, CC, OB, 0) MX_FWD_CASE(DD, CC, OB, 2) MX_FWD_CASE(DD, CC, OB, 3) MX_FWD_CASE(DD, CC, OB, 4)
  MX_FWD_FMTS(64, false, false) MX_FWD_FMTS(64, false, true) MX_FWD_FMTS(64, true, false) MX_FWD_FMTS(64, true, true)
  MX_FWD_FMTS(128, false, false) MX_FWD_FMTS(128, false, true) MX_FWD_FMTS(128, true, false) MX_FWD_FMTS(128, true, true)
#undef MX_FWD_FMTS
#undef MX_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace mxk
