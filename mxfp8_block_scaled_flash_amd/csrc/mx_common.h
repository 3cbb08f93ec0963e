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

// 2^(k-127) as an fp32 value, for k in [1, 254].
MX_DEV float e8m0_f32(int k) { return __uint_as_float((uint32_t)k << 23); }

MX_DEV float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
MX_DEV float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
MX_DEV uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

MX_DEV float wave_max_xor(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }

}  // namespace mxk
