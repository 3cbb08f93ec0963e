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
//     tensors, and zero the fp16 dQ accumulator (head-major [H, T, D], so a
//     head's rows are contiguous for the atomics).
//  2. attn_bwd_kernel: one workgroup per (sequence, head, 256-key tile),
//     eight waves of 32 keys, walking 64-query tiles.  Per tile each wave
//     computes S = Q^ K^T and dP = dO^ V^T (scaled MFMA, keys as the output
//     columns so a lane owns one key), p = exp2(S c - LSE log2 e),
//     dS = p (dP - D), then MX codes of P (32 queries per key) and of dS
//     (square 32 x 32 blocks, wave-wide amax), and accumulates dV^T and
//     dK^T in registers.  The dS codes go to LDS, and the workgroup's waves
//     then form dQ = dS K for the tile (256 keys of contraction) and add it,
//     scaled by softmax_scale * 2^s, into the fp16 accumulator with packed
//     fp16 atomics laid along contiguous features (neighbouring lanes pair
//     up), so each atomic instruction touches four 64-byte row segments.  Q^ and dO^ are read from LDS in both
//     orientations: rows as MFMA operands, columns through
//     ds_read_b64_tr_b8 (one payload, both GEMMs).
//  3. bwd_dq_kernel: dQ = acc * 2^-s in the output type.
#include <type_traits>

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

// The same with element formats fa, fb for the two operands (0 E4M3, 2 E2M3, 3 E3M2, 4 E2M1).
template <int FA, int FB, int OA, int OB>
MX_DEV v16f mfma32f(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, OA, sa, OB, sb);
}

// One 32-element block of a small-format operand: 24 (6-bit) or 16 (4-bit) packed bytes, as the
// instruction reads them from the first dwords of the operand.
template <int W>
MX_DEV v8i small_operand(const uint8_t* p) {
  if constexpr (W == 6) {
    const uint2 x = ((const uint2*)p)[0], y = ((const uint2*)p)[1], z = ((const uint2*)p)[2];
    return v8i{(int)x.x, (int)x.y, (int)y.x, (int)y.y, (int)z.x, (int)z.y, 0, 0};
  } else {
    const uint4 x = *(const uint4*)p;
    return v8i{(int)x.x, (int)x.y, (int)x.z, (int)x.w, 0, 0, 0, 0};
  }
}

MX_DEV v2i tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((v2i __attribute__((address_space(3)))*)(p));
}

// A 64-deep operand whose K index runs down rows {0..15} (block 0) and 32 + {0..15} (block 1) of
// a byte tile, lane column lane % 32 of the chosen 32 columns: four transpose reads, lane (G, i16) =
// (lane / 16, lane % 16) reading 8 bytes of row 16 (G / 2) + i16 / 2 (+ 8, 32, 40).
//
// Over an unpadded 64-byte-row tile whose 16-byte chunks sit XOR-swizzled by (row & 3); chunk0 =
// the operand's first chunk (2 t for query block t).  Rows r, r+8, r+32, r+40 share r & 3.
MX_DEV v8i tr_operand_swz64(const uint8_t* rows, int chunk0, int lane) {
  const int G = lane >> 4, i16 = lane & 15;
  const int r = 16 * (G >> 1) + (i16 >> 1);
  const uint8_t* p = rows + r * 64 + 16 * ((chunk0 + (G & 1)) ^ (r & 3)) + 8 * (i16 & 1);
  v2i r0 = tr8(p), r1 = tr8(p + 8 * 64), r2 = tr8(p + 32 * 64), r3 = tr8(p + 40 * 64);
  return v8i{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// The same four transpose reads from a lane's first row address p (row 16 (G / 2) + i16 / 2 of the
// operand, bytes 16 (G & 1) + 8 (i16 & 1) of its 32 columns), the rows 8, 32 and 40 further down at
// byte offsets O8, O32, O40 (O8 = 8 x stride etc. for equally spaced rows).
template <int O8, int O32, int O40>
MX_DEV v8i tr_operand_rows(const uint8_t* p) {
  v2i r0 = tr8(p), r1 = tr8(p + O8), r2 = tr8(p + O32), r3 = tr8(p + O40);
  return v8i{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// Paired-row layouts of the E4M3 K, Q and dO tiles at D = 128: rows 2j and 2j + 1 adjacent, two
// spare 16-byte slots after each pair (the 144-byte average of a padded row), and one more slot
// shifting every other 8-row (K) or 16-row (Q, dO) group by 16 bytes.  A transpose read pass
// (8 consecutive rows, 32 bytes each) then covers all 64 banks once, and so does a row read pass
// (16 lanes, 16 bytes each) over the rows the lanes read: 16 consecutive keys of K, or the 16
// permuted query rows {0..7, 16..23} (and {8..15, 24..31}) of Q and dO.  With 144-byte rows the
// transpose reads hit bank pairs twice (measured 1.78 against 1.36 ns per read).  Slot of row r
// from the tile start:
MX_DEV constexpr int krow_slot(int r) { return 8 * r + 2 * (r >> 1) + ((r >> 3) & 1); }
MX_DEV constexpr int qrow_slot(int r) { return 8 * r + 2 * (r >> 1) + ((r >> 4) & 1); }
// rows r, r + 8, r + 32, r + 40 for the transpose reads' first rows r (r % 16 < 8)
static_assert(krow_slot(8) - krow_slot(0) == 73 && krow_slot(24) - krow_slot(16) == 73 && krow_slot(32) == 288 &&
              krow_slot(47) - krow_slot(7) == 361 && krow_slot(64) == 576, "K row slots");
static_assert(qrow_slot(8) - qrow_slot(0) == 72 && qrow_slot(31) - qrow_slot(23) == 72 && qrow_slot(32) == 288 &&
              qrow_slot(63) - qrow_slot(23) == 360 && qrow_slot(64) == 576, "Q row slots");

// The dS code tile [key][query] (E4M3 and MXFP4 Q, K): 64-byte rows with 32 spare bytes after every fourth, so
// row r starts at 64 r + 32 (r >> 2).  A transpose read pass (8 consecutive rows, 32 bytes of
// each) then covers all 64 banks once (80-byte rows: 1.80 ns per read, a conflict-free pass 1.34),
// and every address of the tile stays a lane offset plus constants.
constexpr int kDsGroupBytes = 4 * 64 + 32;
MX_DEV constexpr int ds_row(int r) { return 64 * r + 32 * (r >> 2); }

// 64-deep operand whose K index runs down rows {0..15} and 32 + {0..15} of such a tile from row
// 0 of `base` (a multiple of 8), lane column `col0 + lane % 32`: four transpose reads.
MX_DEV v8i tr_operand_ds(const uint8_t* base, int col0, int lane) {
  const int G = lane >> 4, i16 = lane & 15;
  const uint8_t* p = base + ds_row(16 * (G >> 1) + (i16 >> 1)) + col0 + 16 * (G & 1) + 8 * (i16 & 1);
  v2i r0 = tr8(p), r1 = tr8(p + ds_row(8)), r2 = tr8(p + ds_row(32)), r3 = tr8(p + ds_row(40));
  return v8i{r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

MX_DEV uint32_t ld_scale_word(const uint8_t* p, int nbytes) {
  return nbytes == 4 ? *(const uint32_t*)p : *(const uint16_t*)p;
}

typedef _Float16 h2v __attribute__((ext_vector_type(2)));

// Packed fp16 atomic add through a buffer resource (buffer_atomic_pk_add_f16): a 32-bit byte
// offset from a scalar base, its wave-uniform part in an SGPR (soffset), so per-element constants
// cost no vector registers.
MX_DEV void atomic_add_h2_buf(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint32_t uniform_off, float a, float b) {
  h2v v = {(_Float16)a, (_Float16)b};
  __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_v2f16(v, r, (int)byte_off, (int)__builtin_amdgcn_readfirstlane(uniform_off), 0);
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
    // zero this row's fp16 dQ accumulator (D halves; the accumulator is head-major [H, T, D]),
    // when the caller's path has one, and clear the range flag
    if (a.acc) {
      if (row == 0 && c == 0) *a.ovf = 0u;
      uint4 z = make_uint4(0, 0, 0, 0);
      uint16_t* accp = (uint16_t*)a.acc + ((row % a.H) * (long)a.T + row / a.H) * D;
      for (int i = c; i < D / 8; i += LPR) *(uint4*)(accp + i * 8) = z;
    }
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
// One workgroup of eight waves per (sequence, head, 256-key tile), walking
// 64-query steps.  The dQ atomics execute at the memory side (the counters
// show none performed in the per-XCD L2s); their volume -- one fp16 partial
// per key tile and query -- bounded this kernel at 128-key tiles; 256-key
// tiles halve it, and the staggered dQ phase hides most of what remains.
// Wave w owns key block w (32 keys; lane = one key) for the whole walk:
//  A. per query block t = 0, 1: S = Q^ K^T and dP = dO^ V^T (keys as the
//     output columns), p and dS, their MX codes (P: one scale per key and 32
//     queries; dS: one scale per square 32 x 32 block), kept in registers as
//     the B operands below; the dS codes also go to LDS as [key][query];
//  B. dV^T += dO^T P^ and dK^T += Q^T dS^ for its keys and all D features
//     (contraction over the 64 queries; Q^T, dO^T through transpose reads);
//  C. wave w < 2D/32 forms one 32 x 32 (query block, feature chunk) tile of
//     dQ = dS^ K^ over the 256 keys for the previous step (whose dS codes
//     every wave finished before this step began; the dS tile is
//     double-buffered by step) and adds it to the fp16 accumulator with
//     packed atomics.
// The next step's Q^ / dO^ tiles go by DMA (buffer loads with the LDS as
// destination) into the other LDS buffer during the step, its scales, LSE and
// D through registers stored at the step's end: one barrier per step.  Waves 0-3 run C at the start of the step and waves 4-7 at its
// end: the two waves sharing a SIMD (w and w + 4) are then in different
// phases, so one's matrix products overlap the other's elementwise work
// instead of both waiting on the same unit (measured: 10.9 -> 10.0 ms).
// The two halves run separate copies of the step loop, and only waves 0-3
// issue the next step's loads: a wave's waits on its own loads also wait on
// the atomics it issued after them, so waves 4-7, whose atomics come last,
// load nothing and reach the barrier without waiting on memory.
template <int D, bool CAUSAL, int QF>
__global__ __launch_bounds__(512) void attn_bwd_kernel(BwdArgs a) {
  // QF: element format of Q and K (0: MXFP8 E4M3; 2, 3: MXFP6 E2M3, E3M2; 4: MXFP4 E2M1).  In the small
  // formats (D = 128 only) Q and K arrive row-packed (S = Q^ K^T) and column-packed (dK = dS^T Q^ and
  // dQ = dS^ K^ contract over tokens), and the V tile drops its padding for XOR-swizzled chunks so
  // the larger tiles fit in LDS (so does MXFP6's dS tile; MXFP4's keeps the E4M3 layout).  MXFP6 K rows (96 bytes, read as three 8-byte pieces, 32
  // lanes a pass) sit 104 bytes apart, stored through registers, so a pass hits distinct banks (at
  // 96 bytes lanes share bank pairs, 2.4x the time per read; the backward took 7% longer); the DMA'd MXFP6 Q rows
  // stay unpadded (a 16-byte spare slot does not fit in the LDS), as do the 64-byte MXFP4 rows (80-byte
  // rows measured 4% slower overall).
  constexpr bool SMALL = QF != 0;
  constexpr int W = QF == 0 ? 8 : QF == 4 ? 4 : 6;   // bits per Q / K element
  constexpr int BB = 32 * W / 8;                     // bytes of one packed 32-element block
  constexpr int KRB = D * W / 8;                     // bytes of one packed Q / K row
  static_assert(!SMALL || D == 128, "small-format Q, K for D = 128 only");
  constexpr int NW = 8;
  constexpr int BN = 32 * NW;   // keys per workgroup
  constexpr int BQ = 64;        // queries per step
  constexpr int NC = D / 64;    // 64-feature chunks of the S / dP contraction
  constexpr int ND = D / 32;    // 32-feature chunks of dK, dV, dQ
  constexpr int NB = D / 32;    // scale bytes per SQ32 / ROW32 scale word
  constexpr int KST = D + 16;   // LDS row stride of the V tile, and of K, Q, dO where not paired (below)
  constexpr int NT = NW * 64;
  constexpr int SLQ = KST / 16;                 // 16-byte slots per padded Q / dO row
  constexpr int NBQ = BQ * KST / 1024;          // 1 KB DMA blocks per tile (one wave instruction each)
  static_assert(BQ * KST % 1024 == 0, "tiles must be whole DMA blocks");
  constexpr bool PAIRED = !SMALL && D == 128;   // paired-row K, Q, dO tiles (krow_slot, qrow_slot)
  // byte offsets of rows 8, 32, 40 past a transpose read's first row
  constexpr int KO8 = PAIRED ? 16 * 73 : 8 * KST, KO32 = 32 * (PAIRED ? 144 : KST), KO40 = PAIRED ? 16 * 361 : 40 * KST;
  constexpr int QO8 = PAIRED ? 16 * 72 : 8 * KST, QO32 = 32 * (PAIRED ? 144 : KST), QO40 = PAIRED ? 16 * 360 : 40 * KST;
  // the dO tile at D = 128 is paired too: like Q for E4M3 (permuted rows), like K (krow_slot) for
  // MXFP6, whose lanes read its rows in natural order (11.5 -> 11.1 ms); MXFP4 keeps the padded
  // rows (paired: 9.35 -> 9.47 ms, its spills 7 -> 11)
  constexpr bool DOPAIR = D == 128 && (!SMALL || W == 6);
  constexpr int DO8 = !DOPAIR ? QO8 : SMALL ? 16 * 73 : 16 * 72, DO32 = 32 * (DOPAIR ? 144 : KST),
                DO40 = !DOPAIR ? QO40 : SMALL ? 16 * 361 : 16 * 360;
  constexpr int VST = SMALL ? D : KST;          // V row stride (small formats: chunk j of row r in slot j ^ (r & 7))
  // dS code tile: 64-byte rows with a spare half row after every fourth (ds_row), or, where that
  // does not fit in the LDS (MXFP6), unpadded rows with chunk j in slot j ^ (r & 3)
  constexpr bool DSPAD = !(SMALL && W == 6);
  constexpr int DST = BQ;
  constexpr int DSB = DSPAD ? BN / 4 * kDsGroupBytes : BN * DST;   // dS code tile bytes
  constexpr int KRS = W == 6 ? 104 : KRB;       // small formats: LDS row stride of the packed K rows
  constexpr int QRS = KRB;                      // small formats: LDS row stride of the packed Q rows
  constexpr int KROW = SMALL ? BN * KRS : BN * KST;   // row-major K tile bytes
  constexpr int KCOL = SMALL ? (BN / 32) * D * BB : 0;   // column-packed K: [key block][feature][BB]
  constexpr int QROW = SMALL ? BQ * QRS : BQ * KST;   // row-major Q step tile bytes
  constexpr int QCOL = SMALL ? 2 * D * BB : 0;        // column-packed Q: [query block][feature][BB]
  constexpr int NBQR = QROW / 1024, NBQC = QCOL / 1024;   // DMA blocks of the Q tiles
  constexpr int NBDO = BQ * KST / 1024;                   // DMA blocks of the dO tile
  constexpr int NBT = NBQR + NBQC + NBDO;                 // DMA blocks per step (Q, then dO)
  static_assert(QROW % 1024 == 0 && QCOL % 1024 == 0 && (D * BB) % 1024 == 0, "tiles must be whole DMA blocks");
  __shared__ __attribute__((aligned(16))) uint8_t sK[KROW + KCOL];
  __shared__ __attribute__((aligned(16))) uint8_t sV[BN * VST];
  // Q^ and dO^ step tiles arrive by 16-byte DMA (buffer loads straight into LDS): a padded row
  // is KST / 16 slots, the last one a copy of the row's last chunk (never read); in the paired layout
  // (E4M3, D = 128) the spare slots hold copies too
  __shared__ __attribute__((aligned(1024))) uint8_t sQ[2][QROW + QCOL];
  __shared__ __attribute__((aligned(1024))) uint8_t sDO[2][BQ * KST];
  __shared__ __attribute__((aligned(16))) uint8_t sDS[2][DSB];   // [step parity]
  __shared__ uint32_t sKs[NW];                 // K SQ32 scale word (bytes = feature blocks) per key block
  __shared__ uint32_t sVs[BN];                 // V ROW32 scale word per key
  __shared__ uint32_t sQs[2][2], sDOs[2][2];   // [buffer][query block]
  __shared__ __attribute__((aligned(16))) float sL[2][BQ];    // LSE log2(e)
  __shared__ __attribute__((aligned(16))) float sDv[2][BQ];   // D
  __shared__ int sDSs[2][2][NW];               // dS scale code of [step parity][query block][key block]

  saturating_fp8_converts();
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, n = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int id = blockIdx.x, xcd = id & 7, jj = id >> 3;
  const int u = (jj / a.nkt) * 8 + xcd;
  if (u >= a.nseq * a.H) return;
  const int kt = jj % a.nkt;          // low key tiles see the most queries under causality: first
  const int h = __builtin_amdgcn_readfirstlane(u % a.H), s = __builtin_amdgcn_readfirstlane(u / a.H);
  int tok0, L, srow0, sblk0;
  a.seq.get(s, tok0, L, srow0, sblk0);
  tok0 = __builtin_amdgcn_readfirstlane(tok0);   // wave-uniform (from the workgroup index)
  L = __builtin_amdgcn_readfirstlane(L);
  srow0 = __builtin_amdgcn_readfirstlane(srow0);
  sblk0 = __builtin_amdgcn_readfirstlane(sblk0);
  const int kbase = kt * BN;
  if (kbase >= L) return;
  const long rowH = (long)a.H * D;
  const int kw0 = kbase + 32 * w;     // this wave's key block
  const int kj = kw0 + n;             // this lane's key

  // ---- K and V tiles (zero past the end) and their scales
  if constexpr (!SMALL) {
    for (int ch = tid; ch < BN * D / 16; ch += NT) {
      const int r = ch / (D / 16), cx = ch % (D / 16);
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (kbase + r < L) {
        const long off = (long)(tok0 + kbase + r) * rowH + (long)h * D + cx * 16;
        kv = *(const uint4*)(a.k + off);
        vv = *(const uint4*)(a.v + off);
      }
      *(uint4*)(sK + (PAIRED ? 16 * krow_slot(r) : r * KST) + cx * 16) = kv;
      *(uint4*)(sV + r * KST + cx * 16) = vv;
    }
  } else {
    for (int ch = tid; ch < BN * D / 16; ch += NT) {   // V: swizzled, unpadded
      const int r = ch / (D / 16), cx = ch % (D / 16);
      uint4 vv = make_uint4(0, 0, 0, 0);
      if (kbase + r < L) vv = *(const uint4*)(a.v + (long)(tok0 + kbase + r) * rowH + (long)h * D + cx * 16);
      *(uint4*)(sV + r * VST + 16 * (cx ^ (r & 7))) = vv;
    }
    const long rowHk = (long)a.H * KRB;
    for (int ch = tid; ch < BN * KRB / 16; ch += NT) {   // K rows, packed
      const int r = ch / (KRB / 16), cx = ch % (KRB / 16);
      uint4 kv = make_uint4(0, 0, 0, 0);
      if (kbase + r < L) kv = *(const uint4*)(a.k + (long)(tok0 + kbase + r) * rowHk + (long)h * KRB + cx * 16);
      if constexpr (KRS % 16 != 0) {   // 104-byte rows: 8-byte aligned
        uint2* d = (uint2*)(sK + r * KRS + cx * 16);
        d[0] = make_uint2(kv.x, kv.y);
        d[1] = make_uint2(kv.z, kv.w);
      } else {
        *(uint4*)(sK + r * KRS + cx * 16) = kv;
      }
    }
    for (int ch = tid; ch < KCOL / 16; ch += NT) {     // K columns, packed per key block
      const int kb = ch / (D * BB / 16), cx = ch % (D * BB / 16);
      uint4 kv = make_uint4(0, 0, 0, 0);
      if (kbase + 32 * kb < L)
        kv = *(const uint4*)(a.kc + ((long)(sblk0 + kbase / 32 + kb) * a.H + h) * (D * BB) + cx * 16);
      *(uint4*)(sK + KROW + kb * (D * BB) + cx * 16) = kv;
    }
  }
  if (tid < NW) {
    uint32_t wk = 0;
    if (kbase + 32 * tid < L) wk = ld_scale_word(a.ks + ((long)(sblk0 + kbase / 32 + tid) * a.H + h) * NB, NB);
    sKs[tid] = wk;
  }
  for (int r = tid; r < BN; r += NT)
    sVs[r] = (kbase + r < L) ? ld_scale_word(a.vs + ((long)(srow0 + kbase + r) * a.H + h) * NB, NB) : 0u;

  // ---- staging of one query step
  struct Stage {
    float l, d;
    uint32_t qs, dos;
  };
  auto lse_index = [&](int q) -> long {
    return a.seq.cu ? (long)h * a.T + tok0 + q : ((long)s * a.H + h) * a.seq.S + q;
  };
  // Per-step buffer resources end with the sequence: rows, LSE/D entries and
  // scale blocks past its end read as zero (masked later), with no clamps.
  // the step's Q^ / dO^ tiles go to LDS buffer buf by DMA (lane l of an instruction fills bytes
  // 16 l .. 16 l + 15 of its 1 KB block); LSE, D and the scales are loaded into registers
  auto load_step = [&](int q0, int buf, Stage& st, auto dma_waves) {
    constexpr int DW = decltype(dma_waves)::value;   // waves 0 .. DW-1 share the DMA
    const int rows = min(BQ, L - q0);   // >= 1
    const long tb = (long)(tok0 + q0) * rowH + (long)h * D;
    const int nrec = (rows - 1) * (int)rowH + D;
    const __amdgpu_buffer_rsrc_t rdo = buffer_rsrc(a.dob + tb, nrec);
    if constexpr (!SMALL) {
      const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(a.q + tb, nrec);
#pragma unroll
      for (int j = 0; j < (2 * NBQ + DW - 1) / DW; ++j) {
        const int blk = w + DW * j;               // Q blocks first, then dO
        if (w < DW && (2 * NBQ % DW == 0 || blk < 2 * NBQ)) {
          const bool isq = blk < NBQ;
          const int b = isq ? blk : blk - NBQ;
          const int ch = b * 64 + lane;   // 16-byte slot of the tile
          int r, c;
          if constexpr (PAIRED) {
            // the row and chunk of slot ch (qrow_slot inverted: 32-row halves of 288 slots, rows 16-31
            // of a half from slot 145, pairs of rows 18 slots apart); spare slots load a copy
            const int hf = ch / 288, s1 = ch - 288 * hf;
            const int up = s1 >= 144 ? 1 : 0;
            const int u = max(s1 - 145 * up, 0);
            const int pr = u / 18, o = min(u - 18 * pr, 15);
            r = 32 * hf + 16 * up + 2 * pr + (o >> 3);
            c = o & 7;
          } else {
            r = ch / SLQ;
            c = min(ch % SLQ, D / 16 - 1);
          }
          const int off = r * (int)rowH + 16 * c;
          uint8_t* dst = (isq ? sQ[buf] : sDO[buf]) + 1024 * b;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(isq ? rq : rdo, (__attribute__((address_space(3))) void*)dst, 16,
                                                   off, 0, 0, 0);
        }
      }
    } else {
      // packed Q rows (rows contiguous in LDS), then the column-packed blocks of the step's two query
      // blocks (each D BB contiguous bytes), then dO as above
      const long rowHq = (long)a.H * KRB;
      const __amdgpu_buffer_rsrc_t rq =
          buffer_rsrc(a.q + (long)(tok0 + q0) * rowHq + (long)h * KRB, (rows - 1) * (int)rowHq + KRB);
      const int nqb = (rows + 31) / 32;
      const __amdgpu_buffer_rsrc_t rqc = buffer_rsrc(a.qc + ((long)(sblk0 + q0 / 32) * a.H + h) * (D * BB),
                                                     (nqb - 1) * a.H * (D * BB) + D * BB);
#pragma unroll
      for (int j = 0; j < (NBT + DW - 1) / DW; ++j) {
        const int blk = w + DW * j;
        if (w < DW && (NBT % DW == 0 || blk < NBT)) {
          __amdgpu_buffer_rsrc_t r = rdo;
          int off;
          uint8_t* dst;
          if (blk < NBQR) {
            const int p = 16 * (blk * 64 + lane);
            r = rq;
            off = (p / KRB) * (int)rowHq + p % KRB;
            dst = sQ[buf] + 1024 * blk;
          } else if (blk < NBQR + NBQC) {
            const int bb = blk - NBQR, t = bb / (D * BB / 1024);
            r = rqc;
            off = t * a.H * (D * BB) + (bb % (D * BB / 1024)) * 1024 + 16 * lane;
            dst = sQ[buf] + QROW + 1024 * bb;
          } else {
            const int b = blk - NBQR - NBQC;
            const int ch = b * 64 + lane;
            if constexpr (DOPAIR) {
              // the row and chunk of slot ch of the paired dO tile (krow_slot inverted: groups of 8
              // rows, 72 slots each, odd groups from one slot later; pairs of rows 18 slots apart)
              const int gk = ch / 72;
              const int u = max(ch - 72 * gk - (gk & 1), 0);
              const int pr = u / 18, o = min(u - 18 * pr, 15);
              off = (8 * gk + 2 * pr + (o >> 3)) * (int)rowH + 16 * (o & 7);
            } else {
              off = (ch / SLQ) * (int)rowH + 16 * min(ch % SLQ, D / 16 - 1);
            }
            dst = sDO[buf] + 1024 * b;
          }
          __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0, 0);
        }
      }
    }
    // LSE and D by wave 0, the scales by wave 1: the waves that store them
    st = Stage{0.f, 0.f, 0u, 0u};
    if (w == 0) {
      const long li = lse_index(q0);
      st.l = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(a.lse + li, rows * 4), lane * 4, 0, 0));
      st.d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(a.Dbuf + li, rows * 4), lane * 4, 0, 0));
    } else if (w == 1) {
      const long so = ((long)(sblk0 + q0 / 32) * a.H + h) * NB;
      const int snrec = ((rows + 31) / 32 - 1) * a.H * NB + NB;
      const int soff = (lane & 1) * a.H * NB;
      if constexpr (NB == 4) {
        st.qs = __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(a.qs + so, snrec), soff, 0, 0);
        st.dos = __builtin_amdgcn_raw_buffer_load_b32(buffer_rsrc(a.dos + so, snrec), soff, 0, 0);
      } else {
        st.qs = __builtin_amdgcn_raw_buffer_load_b16(buffer_rsrc(a.qs + so, snrec), soff, 0, 0);
        st.dos = __builtin_amdgcn_raw_buffer_load_b16(buffer_rsrc(a.dos + so, snrec), soff, 0, 0);
      }
    }
  };
  auto store_step = [&](int buf, const Stage& st) {
    if (w == 0) {
      sL[buf][lane] = st.l * 1.44269504088896340736f;
      sDv[buf][lane] = st.d;
    } else if (w == 1 && lane < 2) {
      sQs[buf][lane] = st.qs;
      sDOs[buf][lane] = st.dos;
    }
  };

  v16f dvt[ND], dkt[ND];   // dV^T, dK^T: element e = feature 32 dc + 8(e/4) + 4g + e%4, key kj
#pragma unroll
  for (int dc = 0; dc < ND; ++dc) {
    dvt[dc] = v16f{};
    dkt[dc] = v16f{};
  }
  const float cl = a.c;
  const int qstart = CAUSAL ? (kbase / BQ) * BQ : 0;
  const int nsteps = (L - qstart + BQ - 1) / BQ;
  // scale operands of the last dV / dK products, pinned until those products finish
  uint32_t dow_prev = 0, qw_prev = 0;
  int psc_prev = 0, ssc_prev = 0;

  {
    Stage st0;
    load_step(qstart, 0, st0, std::integral_constant<int, NW>{});
    store_step(0, st0);
  }
  __syncthreads();

  // lane offsets of the transpose reads' first rows (row 16 (G / 2) + i16 / 2, bytes 16 (G & 1) + 8 (i16 & 1))
  const int trl = 16 * (lane >> 5) + ((lane & 15) >> 1), trb = 16 * ((lane >> 4) & 1) + 8 * (lane & 1);
  const int trk = (PAIRED ? 16 * krow_slot(trl) : trl * KST) + trb;
  const int trq = (PAIRED ? 16 * qrow_slot(trl) : trl * KST) + trb;
  const int trdo = (DOPAIR ? 16 * (SMALL ? krow_slot(trl) : qrow_slot(trl)) : trl * KST) + trb;

  // ---- C. dQ tile (query block t, feature chunk dc) = (w / ND, w % ND) over the 256 keys of the step
  // at q0, from dS buffer bufc, into the head-major fp16 accumulator [H, T, D] (a head's rows are
  // contiguous).  Output element e of lane l: query 32t + 8(e/4) + 4g + e%4, feature 32 dc + l%32.
  auto phase_c = [&](const int q0, const int bufc) {
    if (w < 2 * ND) {
      const int t = w / ND, dc = w % ND;
      if (q0 + 32 * t < L) {
        v16f acc = v16f{};
        int kscale[BN / 64], sscale[BN / 64];
        // all operands first, then the four products: one LDS round trip instead of four.  Key
        // blocks after every query of the block carry zero dS codes (masked or cleared in A), so
        // they are multiplied in rather than branched around.
        v8i sbv[BN / 64], kav[BN / 64];
#pragma unroll
        for (int kk = 0; kk < BN / 64; ++kk) {
          sscale[kk] = sDSs[bufc][t][2 * kk + g];
          kscale[kk] = (int)((sKs[2 * kk + g] >> (8 * dc)) & 0xFFu);
          if constexpr (DSPAD)
            sbv[kk] = tr_operand_ds(sDS[bufc] + ds_row(64 * kk), 32 * t, lane);   // rows: queries, K: keys
          else
            sbv[kk] = tr_operand_swz64(sDS[bufc] + (64 * kk) * DST, 2 * t, lane);
          if constexpr (!SMALL) {
            kav[kk] = tr_operand_rows<KO8, KO32, KO40>(sK + (PAIRED ? 16 * krow_slot(64 * kk) : 64 * kk * KST) + 32 * dc +
                                                       trk);   // columns: features
          } else {
            // column-packed K: key block 2 kk + g of feature 32 dc + n
            kav[kk] = small_operand<W>(sK + KROW + ((2 * kk + g) * D + 32 * dc + n) * BB);
          }
        }
#pragma unroll
        for (int kk = 0; kk < BN / 64; ++kk) acc = mfma32f<0, QF, 0, 0>(sbv[kk], kav[kk], acc, sscale[kk], kscale[kk]);
        keep(acc[0]);
#pragma unroll
        for (int kk = 0; kk < BN / 64; ++kk) {
          keep(kscale[kk]);
          keep(sscale[kk]);
        }
        // packed fp16 atomics, neighbouring lanes paired: the even lane of a pair adds (row r,
        // features f, f+1) of element e, the odd lane (row r + 1, features f-1, f) of element e + 1
        const int odd = lane & 1;
        _Float16* abase = (_Float16*)a.acc + (((long)h * a.T + tok0 + q0 + 32 * t) * D + 32 * dc);
        const uint32_t rh = (uint32_t)D;
        // the tile's 32 rows lie within 32 D halves of abase
        const __amdgpu_buffer_rsrc_t ars = buffer_rsrc(abase, (int)(64u * rh));
        const uint32_t lofs = (uint32_t)(4 * g + odd) * rh + (uint32_t)(n - odd);
        const int rows_left = L - q0 - 32 * t - 4 * g - odd;   // element rows c_e below this are in range
        const float mult = a.dq_mult;
        // a scaled partial beyond fp16's largest finite value would saturate in the convert (the
        // wave's MODE): report it through the range flag instead of passing it on silently
        float big = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) big = fmaxf(big, fabsf(acc[e]));
        if (big * mult > 65504.f) *a.ovf = 1u;
        auto add_tile = [&](auto checked) {
#pragma unroll
          for (int e = 0; e < 16; e += 2) {
            const float x0 = acc[e], x1 = acc[e + 1];
            const float send = odd ? x0 : x1;
            const float got = __int_as_float(
                __builtin_amdgcn_update_dpp(__float_as_int(send), __float_as_int(send), 0xB1, 0xF, 0xF, false));
            const float lo_v = odd ? got : x0, hi_v = odd ? x1 : got;
            const int ce = 8 * (e >> 2) + (e & 3);
            if (!decltype(checked)::value || ce < rows_left)
              atomic_add_h2_buf(ars, 2u * lofs, 2u * (uint32_t)ce * rh, lo_v * mult, hi_v * mult);
          }
        };
        if (q0 + 32 * t + 32 <= L) add_tile(std::false_type{});
        else add_tile(std::true_type{});
      }
    }

  };

  // The step loop in two copies, one per half of the workgroup: waves 0-3 (EARLY) run C first and
  // issue every load of the next step; waves 4-7 run C last and load nothing, so no wait for a
  // load of theirs can hold them behind their own atomics.
  auto walk = [&](auto early) {
    constexpr bool EARLY = decltype(early)::value;
    for (int j = 0; j < nsteps; ++j) {
      const int q0 = qstart + j * BQ, buf = j & 1;
      const uint8_t* sQb = sQ[buf];
      const uint8_t* sDOb = sDO[buf];
      if (EARLY && j > 0) phase_c(q0 - BQ, buf ^ 1);   // half the waves: the previous step's dQ first
      // ---- A. S and dP for (key block w, query block t): element e = query q0 + 32t + 16g + e (E4M3;
      // small formats: q0 + 32t + 8(e/4) + 4g + e%4)
      v8i pB, sB;        // P and dS codes as B operands: bytes 16t + 0..15 = queries 32t + 16g + 0..15
      int kpc[2], ksc2[2];
      const bool live = kw0 < L && !(CAUSAL && kw0 > q0 + BQ - 1);   // a key of the block sees a query
      if (live) {
        const uint8_t* kr = sK + (PAIRED ? 16 * krow_slot(32 * w + n) : (32 * w + n) * KST) + 16 * g;
        const uint8_t* vr = sV + (32 * w + n) * KST + 16 * g;
        // small formats: packed K row of this lane's key (block 2 c + g at (2 c + g) BB); swizzled V row
        const uint8_t* krs = sK + (32 * w + n) * KRS + g * BB;
        const uint8_t* vrs = sV + (32 * w + n) * VST;
        auto vchunk = [&](int j) __attribute__((always_inline)) { return *(const uint4*)(vrs + 16 * (j ^ (n & 7))); };
        const uint32_t ksc = sKs[w] >> (8 * g), vsc = sVs[32 * w + n] >> (8 * g);
        // E4M3: lane n supplies query row qrow of each 32-query block to the S and dP products: output
        // row 8(e/4) + 4g + e%4 then holds query 16g + e, so each lane half's P and dS codes are its
        // 16 consecutive queries, the order the dV / dK products and the dS tile take them in (no
        // lane-half exchange).  The small formats keep the natural rows and exchange the codes (with
        // the permuted rows their spills rose from 15-40 to 49-118 registers).
        constexpr bool QPERM = !SMALL;
        const int qrow = QPERM ? ((((n >> 2) & 1) << 4) | (((n >> 3) & 3) << 2) | (n & 3)) : n;
        // element e of lane half g: query qa0 + qoff + qe(e)
        const int qoff = QPERM ? 16 * g : 4 * g;
        auto qe = [](int e) { return QPERM ? e : 8 * (e >> 2) + (e & 3); };
  #pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int qa0 = q0 + 32 * t;
          const bool act = qa0 < L && !(CAUSAL && kw0 > qa0 + 31);
          const bool edge = !act || qa0 + 31 >= L || kw0 + 31 >= L || (CAUSAL && kw0 + 31 > qa0);
          // element e is query qa0 + qoff + qe(e): visible iff lo <= qe(e) < hi
          const int lo = (!act || kj >= L) ? 64 : (CAUSAL ? kj - qa0 - qoff : -64);
          const int hi = L - qa0 - qoff;
          const uint32_t qsa = sQs[buf][t] >> (8 * g), dsa = sDOs[buf][t] >> (8 * g);
          // computed for every block (rows past either end are zero, so the values are
          // finite); the mask zeroes p and dS where nothing is visible
          const int qro = PAIRED ? 16 * (qrow_slot(qrow) + 288 * t) : (32 * t + qrow) * KST;
          const int doro = DOPAIR ? 16 * ((SMALL ? krow_slot(qrow) : qrow_slot(qrow)) + 288 * t) : qro;
          const uint8_t* qp = sQb + qro + 16 * g;
          const uint8_t* op = sDOb + doro + 16 * g;
          v16f st, dpt;
          if constexpr (!SMALL) {
            st = mfma32b<0, 0>(pack8b(*(const uint4*)qp, *(const uint4*)(qp + 32)),
                               pack8b(*(const uint4*)kr, *(const uint4*)(kr + 32)), v16f{}, qsa, ksc);
            dpt = mfma32b<0, 0>(pack8b(*(const uint4*)op, *(const uint4*)(op + 32)),
                                pack8b(*(const uint4*)vr, *(const uint4*)(vr + 32)), v16f{}, dsa, vsc);
            if constexpr (NC > 1) {
              st = mfma32b<2, 2>(pack8b(*(const uint4*)(qp + 64), *(const uint4*)(qp + 96)),
                                 pack8b(*(const uint4*)(kr + 64), *(const uint4*)(kr + 96)), st, qsa, ksc);
              dpt = mfma32b<2, 2>(pack8b(*(const uint4*)(op + 64), *(const uint4*)(op + 96)),
                                  pack8b(*(const uint4*)(vr + 64), *(const uint4*)(vr + 96)), dpt, dsa, vsc);
            }
          } else {
            // S from the packed rows (lane half g: 32-element block 2 c + g); dP as above with V swizzled
            const uint8_t* qps = sQb + (32 * t + qrow) * QRS + g * BB;
            st = mfma32f<QF, QF, 0, 0>(small_operand<W>(qps), small_operand<W>(krs), v16f{}, qsa, ksc);
            dpt = mfma32b<0, 0>(pack8b(*(const uint4*)op, *(const uint4*)(op + 32)), pack8b(vchunk(g), vchunk(2 + g)),
                                v16f{}, dsa, vsc);
            st = mfma32f<QF, QF, 2, 2>(small_operand<W>(qps + 2 * BB), small_operand<W>(krs + 2 * BB), st, qsa, ksc);
            dpt = mfma32b<2, 2>(pack8b(*(const uint4*)(op + 64), *(const uint4*)(op + 96)),
                                pack8b(vchunk(4 + g), vchunk(6 + g)), dpt, dsa, vsc);
          }
          // ---- p = 2^(S c - LSE log2 e) (0 where masked), dS = p (dP - D); two copies of the
          // pass: with the mask (diagonal, edge or empty blocks) and without.  LSE and D are read
          // four queries at a time, in two halves fenced off from each other (fewer live registers).
          float am = -INFINITY, sm = 0.f;
          auto pass = [&](auto masked) {
  #pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (q == 2) __builtin_amdgcn_sched_barrier(0);
              const float4 l4 = *(const float4*)(&sL[buf][32 * t + qoff + qe(4 * q)]);
              const float4 d4 = *(const float4*)(&sDv[buf][32 * t + qoff + qe(4 * q)]);
              const float lq[4] = {l4.x, l4.y, l4.z, l4.w}, dq[4] = {d4.x, d4.y, d4.z, d4.w};
  #pragma unroll
              for (int r = 0; r < 4; ++r) {
                const int e = 4 * q + r;
                float arg = fmaf(st[e], cl, -lq[r]);
                if constexpr (decltype(masked)::value) {
                  arg = (qe(e) >= lo && qe(e) < hi) ? arg : -INFINITY;
                }
                const float p = __builtin_amdgcn_exp2f(arg);
                const float ds = p * (dpt[e] - dq[r]);
                st[e] = p;
                dpt[e] = ds;
                am = fmaxf(am, arg);
                sm = fmaxf(sm, fabsf(ds));
              }
            }
          };
          if (edge) pass(std::true_type{});
          else pass(std::false_type{});
          const float amax = half_swap_max(am);   // 32 queries of this key
          const float smax = wave_max_nonneg(sm);  // 32 queries x 32 keys
          // S and dP have been read: their products (and every earlier one) are done
          keep(qsa); keep(dsa); keep(ksc); keep(vsc);
          keep(dow_prev); keep(qw_prev); keep(psc_prev); keep(ssc_prev);
          // ---- MX codes (nothing visible: zero codes, scale 1)
          const int kp = exp2_scale_code(amax);
          const int ks2 = max(scale_code(smax), 1);
          const float psc = e8m0_f32(kp), ssc = e8m0_f32(ks2);   // the converts saturate (wave MODE)
          uint32_t pw[4], sw[4];   // dword q holds queries qoff + qe(4q) + 0..3
  #pragma unroll
          for (int q = 0; q < 4; ++q) {
            if constexpr (W != 6) {
              pw[q] = cvt4_scaled_fp8(st[4 * q], st[4 * q + 1], st[4 * q + 2], st[4 * q + 3], psc);
              sw[q] = cvt4_scaled_fp8(dpt[4 * q], dpt[4 * q + 1], dpt[4 * q + 2], dpt[4 * q + 3], ssc);
            } else {
              // MXFP6 Q, K: through the builtins, each started from a zero word (the asm form raised this
              // variant's spills from 40 to 113 registers, +28% time, and starting from a copy of the
              // first input kept 40; the asm form lowers the E4M3 and E2M1 ones, E2M1 -8%, where the
              // builtins spill more)
              v2s z = {0, 0}, y = {0, 0};
              z = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, st[4 * q], st[4 * q + 1], psc, false);
              z = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(z, st[4 * q + 2], st[4 * q + 3], psc, true);
              pw[q] = __builtin_bit_cast(uint32_t, z);
              y = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(y, dpt[4 * q], dpt[4 * q + 1], ssc, false);
              y = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(y, dpt[4 * q + 2], dpt[4 * q + 3], ssc, true);
              sw[q] = __builtin_bit_cast(uint32_t, y);
            }
          }
          // lane half g holds queries 16g + 0..15 of the block, in order (small formats: after swapping
          // lane halves)
          if constexpr (!QPERM) {
            auto a02 = __builtin_amdgcn_permlane32_swap(pw[0], pw[2], false, false);
            auto a13 = __builtin_amdgcn_permlane32_swap(pw[1], pw[3], false, false);
            auto b02 = __builtin_amdgcn_permlane32_swap(sw[0], sw[2], false, false);
            auto b13 = __builtin_amdgcn_permlane32_swap(sw[1], sw[3], false, false);
            pw[0] = a02[0]; pw[1] = a02[1]; pw[2] = a13[0]; pw[3] = a13[1];
            sw[0] = b02[0]; sw[1] = b02[1]; sw[2] = b13[0]; sw[3] = b13[1];
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            pB[4 * t + q] = pw[q];
            sB[4 * t + q] = sw[q];
          }
          if constexpr (DSPAD)
            *(uint4*)(sDS[buf] + ds_row(32 * w + n) + 32 * t + 16 * g) = make_uint4(sw[0], sw[1], sw[2], sw[3]);
          else
            *(uint4*)(sDS[buf] + (32 * w + n) * DST + 16 * ((2 * t + g) ^ (n & 3))) = make_uint4(sw[0], sw[1], sw[2], sw[3]);
          if (lane == 0) sDSs[buf][t][w] = ks2;
          kpc[t] = kp;
          ksc2[t] = ks2;
        }
        // ---- B. dV^T += dO^T P^ and dK^T += Q^T dS^ (rows: features, contraction: the 64 queries;
        // lane half g supplies the scale of query block g)
        const int pscale = g ? kpc[1] : kpc[0];
        const int sscale = g ? ksc2[1] : ksc2[0];
        const uint32_t dow = sDOs[buf][g], qw = sQs[buf][g];
  #pragma unroll
        for (int dc = 0; dc < ND; ++dc) {
          const v8i oa = tr_operand_rows<DO8, DO32, DO40>(sDOb + 32 * dc + trdo);
          // Q^T: the 64 queries of feature 32 dc + n; small formats from the column-packed blocks
          // (lane half g: query block g)
          const v8i qa = SMALL ? small_operand<W>(sQb + QROW + (g * D + 32 * dc + n) * BB)
                               : tr_operand_rows<QO8, QO32, QO40>(sQb + 32 * dc + trq);
          if (dc == 0) { dvt[0] = mfma32b<0, 0>(oa, pB, dvt[0], dow, pscale); dkt[0] = mfma32f<QF, 0, 0, 0>(qa, sB, dkt[0], qw, sscale); }
          if (dc == 1) { dvt[1] = mfma32b<1, 0>(oa, pB, dvt[1], dow, pscale); dkt[1] = mfma32f<QF, 0, 1, 0>(qa, sB, dkt[1], qw, sscale); }
          if constexpr (ND > 2) {
            if (dc == 2) { dvt[2] = mfma32b<2, 0>(oa, pB, dvt[2], dow, pscale); dkt[2] = mfma32f<QF, 0, 2, 0>(qa, sB, dkt[2], qw, sscale); }
            if (dc == 3) { dvt[3] = mfma32b<3, 0>(oa, pB, dvt[3], dow, pscale); dkt[3] = mfma32f<QF, 0, 3, 0>(qa, sB, dkt[3], qw, sscale); }
          }
        }
        dow_prev = dow; qw_prev = qw; psc_prev = pscale; ssc_prev = sscale;
      } else {
        // every key of the block comes after every query of the step: dS is zero
        const uint4 z = make_uint4(0, 0, 0, 0);
        if constexpr (DSPAD) {
          uint8_t* rowp = sDS[buf] + ds_row(32 * w + (lane >> 1)) + 32 * (lane & 1);
          *(uint4*)rowp = z;
          *(uint4*)(rowp + 16) = z;
        } else {
          const int rr = 32 * w + (lane >> 1);
          uint8_t* rowp = sDS[buf] + rr * DST;
          *(uint4*)(rowp + 16 * ((2 * (lane & 1)) ^ (rr & 3))) = z;
          *(uint4*)(rowp + 16 * ((2 * (lane & 1) + 1) ^ (rr & 3))) = z;
        }
        if (lane == 0) {
          sDSs[buf][0][w] = 1;
          sDSs[buf][1][w] = 1;
        }
      }
      // waves 0-3 fetch the next step's operands while waves 4-7 form their dQ tiles (after
      // the last step, the last one is fetched again and its buffer rewritten)
      const int qn = qstart + min(j + 1, nsteps - 1) * BQ;
      if constexpr (EARLY) {
        Stage nx;
        load_step(qn, buf ^ 1, nx, std::integral_constant<int, 4>{});
        store_step(buf ^ 1, nx);
      } else {
        if (j > 0) phase_c(q0 - BQ, buf ^ 1);
      }
      __syncthreads();
    }
  };
  if (w < 4) walk(std::true_type{});
  else walk(std::false_type{});
  phase_c(qstart + (nsteps - 1) * BQ, (nsteps - 1) & 1);

  // ---- epilogue: dK = softmax_scale * dK^T, dV = dV^T, features 32 dc + 8q + 4g + 0..3 of key kj
  keep(dvt[ND - 1][0]);
  keep(dkt[ND - 1][0]);
  keep(dow_prev); keep(qw_prev); keep(psc_prev); keep(ssc_prev);
  if (kj >= L) return;
  const long orow = (long)(tok0 + kj) * rowH + (long)h * D;
#pragma unroll
  for (int dc = 0; dc < ND; ++dc)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int d = 32 * dc + 8 * q + 4 * g;
      const float k0 = dkt[dc][4 * q] * a.sigma, k1 = dkt[dc][4 * q + 1] * a.sigma,
                  k2 = dkt[dc][4 * q + 2] * a.sigma, k3 = dkt[dc][4 * q + 3] * a.sigma;
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
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a, long n8) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;   // 8-element chunk of dQ [T, H, D]
  if (i >= n8) return;
  const long row = i / (D / 8);                          // (token, head) row
  const long src = ((row % a.H) * (long)a.T + row / a.H) * (D / 8) + i % (D / 8);
  const uint4 raw = *((const uint4*)a.acc + src);
  const _Float16* hp = (const _Float16*)&raw;
  // an accumulator at fp16's largest finite magnitude, infinite or NaN has left the range the
  // static scale was meant to keep it in (read off the bits: the kernel is built without NaN
  // semantics)
  const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
  bool out_of_range = false;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    out_of_range |= (w4[j] & 0x7FFFu) >= 0x7BFFu || ((w4[j] >> 16) & 0x7FFFu) >= 0x7BFFu;
  if (out_of_range) *a.ovf = 1u;
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

template __global__ void attn_bwd_kernel<64, true, 0>(BwdArgs);
template __global__ void attn_bwd_kernel<64, false, 0>(BwdArgs);
template __global__ void attn_bwd_kernel<128, true, 0>(BwdArgs);
template __global__ void attn_bwd_kernel<128, false, 0>(BwdArgs);

hipError_t launch_bwd_pre(int D, bool io_f32, const BwdArgs& a, hipStream_t st) {
  const long rows = (long)a.T * a.H;
  if (rows == 0) return hipSuccess;
  const int epc = io_f32 ? 4 : 8;
  const int rpw = 64 / (D / epc);
  const long waves = (rows + rpw - 1) / rpw;
  dim3 g((unsigned)((waves + 3) / 4)), b(256);
  if (D == 64 && !io_f32) bwd_pre_kernel<64, false><<<g, b, 0, st>>>(a);
  else if (D == 64) bwd_pre_kernel<64, true><<<g, b, 0, st>>>(a);
  else if (!io_f32) bwd_pre_kernel<128, false><<<g, b, 0, st>>>(a);
  else bwd_pre_kernel<128, true><<<g, b, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(int D, bool causal, bool io_f32, BwdArgs a, int max_len, hipStream_t st, int qk_fmt) {
  if (qk_fmt != 0 && D != 128) return hipErrorInvalidValue;
  const long rows = (long)a.T * a.H;
  if (rows == 0) return hipSuccess;
  // 1. D_i and zeroed accumulator
  {
    hipError_t e = launch_bwd_pre(D, io_f32, a, st);
    if (e != hipSuccess) return e;
  }
  // 2. main
  {
    constexpr int BN = 256;   // keys per workgroup
    a.nkt = (max_len + BN - 1) / BN;
    const long units = (long)a.nseq * a.H;
    const long grid = ((units + 7) / 8) * 8 * a.nkt;
    dim3 g((unsigned)grid), b(512);
    if (qk_fmt == 0) {
      if (D == 64 && causal) attn_bwd_kernel<64, true, 0><<<g, b, 0, st>>>(a);
      else if (D == 64) attn_bwd_kernel<64, false, 0><<<g, b, 0, st>>>(a);
      else if (causal) attn_bwd_kernel<128, true, 0><<<g, b, 0, st>>>(a);
      else attn_bwd_kernel<128, false, 0><<<g, b, 0, st>>>(a);
    } else {
#define MX_BWDF_CASE(F)                                                   \
  if (qk_fmt == F) {                                                      \
    if (causal) attn_bwd_kernel<128, true, F><<<g, b, 0, st>>>(a);        \
    else attn_bwd_kernel<128, false, F><<<g, b, 0, st>>>(a);              \
  } else
      MX_BWDF_CASE(2) MX_BWDF_CASE(3) MX_BWDF_CASE(4) return hipErrorInvalidValue;
#undef MX_BWDF_CASE
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // 3. dQ = acc * 2^-s
  {
    const long n8 = rows * D / 8;
    dim3 g((unsigned)((n8 + 255) / 256)), b(256);
    if (D == 64) bwd_dq_kernel<64><<<g, b, 0, st>>>(a, n8);
    else bwd_dq_kernel<128><<<g, b, 0, st>>>(a, n8);
    return hipGetLastError();
  }
}

}  // namespace mxk
