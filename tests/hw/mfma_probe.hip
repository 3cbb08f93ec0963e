// Test-only: runs v_mfma_scale_f32_32x32x64_f8f6f4 once per case on caller-laid-out
// lane operands, so a test can compare the oracle's accumulation model with the
// instruction.  Not part of libmxfa.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ void mfma_probe_kernel(const v8i* a, const v8i* b, const int* sa, const int* sb, v16f* c, int ncase) {
  const int cs = blockIdx.x, l = threadIdx.x;
  if (cs >= ncase) return;
  v16f acc = {};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[cs * 64 + l], b[cs * 64 + l], acc, 0, 0, 0, sa[cs * 64 + l],
                                                        0, sb[cs * 64 + l]);
  c[cs * 64 + l] = acc;
}

// a_lanes, b_lanes: [ncase][64 lanes][32 bytes]; sa, sb: [ncase][64]; out: [ncase][64][16] (device pointers)
extern "C" int mfma_probe(const void* a_lanes, const void* b_lanes, const int* sa, const int* sb, float* out,
                          int ncase) {
  if (ncase <= 0) return 0;
  mfma_probe_kernel<<<ncase, 64>>>((const v8i*)a_lanes, (const v8i*)b_lanes, sa, sb, (v16f*)out, ncase);
  return hipDeviceSynchronize() == hipSuccess ? 0 : 1;
}
