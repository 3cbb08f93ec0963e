// Internal device helpers shared by the MX kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define MX_DEV __device__ __forceinline__

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));

namespace mxk {

constexpr int kBlock = 32;  // elements per MX block

// Where sequence s lives.  Fixed-length tensors are B sequences of S tokens
// each; jagged tensors take the offsets from device arrays.
struct SeqMap {
  const int32_t* cu;    // token offsets [nseq+1] (nullptr: fixed length)
  const int32_t* csr;   // padded scale-row offsets [nseq+1] (varlen only)
  int S;                // fixed length
  int nblk;             // ceil(S/32) for fixed length
  MX_DEV void get(int s, int& tok0, int& L, int& srow0, int& sblk0) const {
    if (cu) {
      tok0 = cu[s];
      L = cu[s + 1] - tok0;
      srow0 = csr[s];
      sblk0 = srow0 >> 5;
    } else {
      tok0 = s * S;
      L = S;
      srow0 = tok0;
      sblk0 = s * nblk;
    }
  }
};

// E8M0 code of a block from its (non-negative) amax: clamp(floor(log2 amax) - 8 + 127, 0, 254),
// read off the fp32 exponent field; zero and subnormal amax give 0.
MX_DEV int scale_code(float amax) {
  int e = (int)(__float_as_uint(amax) >> 23) & 0xFF;
  return max(e - 8, 0);
}

// E8M0 code of a block of values p = fl32(2^a), from the block's largest
// exponent a_max alone: the code clamp(floor(log2 fl32(2^a_max)) + 119, 0, 254)
// that scale_code() would pick from the rounded maximum, raised to at least 1
// (the attention kernels give an empty or fully masked block, code 0, scale 1).
// floor(log2) of the rounded value is floor(a_max), except on
// [log2(1 - 2^-25), 0), where 2^a rounds up to 1.0 (0xB338AA3B is the
// smallest float in that interval, so these are the negative floats whose bit
// patterns lie in [0x80000000, 0xB338AA3B]).  No other fp32 a lies that close
// below an integer.  This makes the decision independent of the accuracy of the
// hardware exp2.  Six VALU instructions: v_cvt_flr_i32_f32 floors and converts
// in one (-inf gives INT_MIN, which the clamp takes to 1); the same codes as
// floor / clamp / convert written out, for every fp32 input but NaN (checked
// exhaustively on the CPU).
MX_DEV int exp2_scale_code(float a_max) {
  int fl;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(fl) : "v"(a_max));
  const bool near_zero = (__float_as_uint(a_max) ^ 0x80000000u) <= 0x3338AA3Bu;   // a_max in [-T, -0]
  const int code = near_zero ? 119 : (int)((uint32_t)fl + 119u);
  return min(max(code, 1), 254);
}

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

// Raw buffer resource over `bytes` bytes from base (untyped accesses; word 3 is
// the gfx9-family default).  Loads past `bytes` return zero.  base and bytes
// must be the same in every lane of the wave: they are read from the first
// lane, so the resource sits in scalar registers.
MX_DEV __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  const uint64_t v = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  void* ub = (void*)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// 2^(k-127) as an fp32 value, for k in [1, 254].
MX_DEV float e8m0_f32(int k) { return __uint_as_float((uint32_t)k << 23); }

// Saturating FP8 converts for this wave: with MODE.FP16_OVFL (bit 23) set, v_cvt_pk_fp8_f32 and
// v_cvt_scalef32_pk_fp8_f32 turn finite values beyond E4M3's range into +-448 (codes 0x7E /
// 0xFE) instead of NaN, the saturating encoding of the OCP MX rules, so no clamp is needed before
// them (measured on gfx950: 465, 1000, 1e10 and -500 give 0x7E / 0xFE; with the bit clear, NaN).
// The bit also makes fp16 results saturate at +-65504 instead of overflowing to infinity.
MX_DEV void saturating_fp8_converts() { __builtin_amdgcn_s_setreg(/* hwreg(HW_REG_MODE, 23, 1) */ 1473, 1); }

MX_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
MX_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
MX_DEV uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

MX_DEV float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }

// Four fp32 values divided by the E8M0 scale `scale` (as fp32) and converted to E4M3 codes, little-
// endian in one dword: two v_cvt_scalef32_pk_fp8_f32 (low, then high half of the dword), written as one
// statement with an early-clobbered output and no tied old value (through the builtin, which ties one,
// the compiler first copied a register into each destination).
MX_DEV uint32_t cvt4_scaled_fp8(float a, float b, float c, float d, float scale) {
  uint32_t r;
  asm("v_cvt_scalef32_pk_fp8_f32 %0, %1, %2, %5\n\tv_cvt_scalef32_pk_fp8_f32 %0, %3, %4, %5 op_sel:[0,0,0,1]"
      : "=&v"(r)
      : "v"(a), "v"(b), "v"(c), "v"(d), "v"(scale));
  return r;
}

// max of v and the value of the lane 32 apart (v_permlane32_swap exchanges the wave's halves)
MX_DEV float half_swap_max(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int CTRL>
MX_DEV int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Wave-wide max of non-negative floats.  Their bit patterns order like the
// values, so the reduction runs on integers: DPP within rows of 16 lanes
// (quad swaps, half-row and row mirrors), then v_permlane16_swap and
// v_permlane32_swap across rows.
MX_DEV float wave_max_nonneg(float f) {
  int v = __float_as_int(f);
  v = max(v, dpp_i32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_i32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_i32<0x141>(v));   // row_half_mirror
  v = max(v, dpp_i32<0x140>(v));   // row_mirror
  auto a = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = max((int)a[0], (int)a[1]);
  auto b = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return __int_as_float(max((int)b[0], (int)b[1]));
}

// The scaled MFMA reads its operand registers (data and E8M0 scales) over the
// passes of the instruction, and the compiler may hand those registers to
// other values as soon as the instruction has issued.  keep() pins values in
// their registers up to a point placed after something that consumes the
// MFMA's result (which waits for the instruction to finish).
template <typename T>
MX_DEV void keep(const T& x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" ::"v"(x));
#endif
}

}  // namespace mxk
