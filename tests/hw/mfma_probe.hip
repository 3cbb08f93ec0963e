// Test and measurement infrastructure, not part of libmxfa:
//  * mfma_probe: runs v_mfma_scale_f32_32x32x64_f8f6f4 once per case on caller-laid-out lane
//    operands, so tests can compare the instruction with the oracle's stated product bound.
//  * mfma_peak: a loop of independent scaled MFMAs per wave (register operands, no memory traffic),
//    the ceiling of the matrix core for this instruction on the device at its sustained clock.
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

// Four independent accumulator chains per wave, `iters` x 4 MFMAs; one float per thread written so
// the products are not dead.  256 threads per block (one wave per SIMD).
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* out) {
  const int l = threadIdx.x;
  v8i a = {l, l + 1, l + 2, l + 3, l + 4, l + 5, l + 6, l + 7};
  v8i b = {l ^ 7, l ^ 5, l ^ 3, l ^ 1, l, l + 9, l + 11, l + 13};
  a &= 0x3F3F3F3F;   // finite E4M3 codes
  b &= 0x3F3F3F3F;
  v16f c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c0, 0, 0, 0, 127, 0, 127);
    c1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, a, c1, 0, 0, 0, 127, 0, 127);
    c2 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, a, c2, 0, 0, 0, 127, 0, 127);
    c3 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b, b, c3, 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * 256 + l] = s;
}

// Runs the peak loop on `blocks` workgroups of 256 threads; returns the kernel time in ms (hip events).
extern "C" float mfma_peak(int iters, int blocks, float* out) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.f;
  mfma_peak_kernel<<<blocks, 256>>>(iters, out);   // warm-up
  hipEventRecord(e0, 0);
  mfma_peak_kernel<<<blocks, 256>>>(iters, out);
  hipEventRecord(e1, 0);
  if (hipEventSynchronize(e1) != hipSuccess) return -1.f;
  float ms = 0.f;
  hipEventElapsedTime(&ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return ms;
}
