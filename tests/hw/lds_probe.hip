// LDS read-pattern probe (measurement infrastructure, run on the GPU by tests/hw/lds_banks.py): every
// wave of every workgroup reads LDS with one instruction kind at per-lane byte offsets from a table
// (the operand-read patterns of the kernels' LDS tiles), eight reads per iteration at eight bases
// 4096 bytes apart; the time per read instruction against the linear pattern shows the pattern's
// bank conflicts.  Offsets are checked by the caller to stay inside the 64 KB buffer
// (offset + read size + 7 * 4096 <= 65536).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v2i __attribute__((ext_vector_type(2)));

namespace {

template <int KIND>   // 0: ds_read_b128, 1: ds_read_b64, 2: ds_read_b64_tr_b8
__global__ __launch_bounds__(512) void lds_read_kernel(const int* pat, uint32_t* out, int iters) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[65536];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < 4096; i += 512) ((uint4*)buf)[i] = make_uint4(i, i * 3, i * 5, i * 7);
  __syncthreads();
  int off = pat[lane];
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
    asm volatile("" : "+v"(off));   // the reads stay in the loop
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint8_t* p = buf + off + 4096 * ((it + u + (tid >> 6)) & 7);
      if constexpr (KIND == 0) {
        const uint4 x = *(const uint4*)p;
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
      } else if constexpr (KIND == 1) {
        const uint2 x = *(const uint2*)p;
        acc ^= x.x ^ x.y;
      } else {
        const v2i x = __builtin_amdgcn_ds_read_tr8_b64_v2i32((v2i __attribute__((address_space(3)))*)(p));
        acc ^= (uint32_t)(x[0] ^ x[1]);
      }
    }
  }
  out[blockIdx.x * 512 + tid] = acc;
}

}  // namespace

// Milliseconds of one launch of `blocks` workgroups (8 waves each, `iters` x 8 reads per wave), or a
// negative value on a HIP error.  pat: 64 device ints; out: blocks * 512 device uint32.
extern "C" float lds_probe(int kind, const int* pat, uint32_t* out, int blocks, int iters) {
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.f;
  hipEventRecord(e0, 0);
  if (kind == 0) lds_read_kernel<0><<<blocks, 512>>>(pat, out, iters);
  else if (kind == 1) lds_read_kernel<1><<<blocks, 512>>>(pat, out, iters);
  else lds_read_kernel<2><<<blocks, 512>>>(pat, out, iters);
  hipEventRecord(e1, 0);
  float ms = -1.f;
  if (hipGetLastError() == hipSuccess && hipEventSynchronize(e1) == hipSuccess) hipEventElapsedTime(&ms, e0, e1);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  return ms;
}
