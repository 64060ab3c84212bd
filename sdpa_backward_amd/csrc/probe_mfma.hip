// Sustained bf16 MFMA throughput of this GPU at the clock it actually runs:
// every wave issues two independent chains of v_mfma_f32_32x32x16_bf16 on
// register operands (no memory traffic inside the loop). The benchmark
// reports its kernels' throughput against the published dense peak and, next
// to it, against this measured ceiling.
#include "sdpa_probe.h"

#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256, 1) mfma_chain_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    a[j] = (__bf16)(0.001f * (lane + j));
    b[j] = (__bf16)(0.002f * (j + 1));
  }
  f32x16 c0 = {}, c1 = {};
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int u = 0; u < 4; u++) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; i++) s += c0[i] + c1[i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int sdpa_probe_mfma_bf16(float* out, int32_t n_workgroups, int32_t iters, hipStream_t stream) {
  if (out == nullptr || n_workgroups <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_chain_kernel, dim3((unsigned)n_workgroups), dim3(256), 0, stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

extern "C" double sdpa_probe_mfma_bf16_flop(int32_t n_workgroups, int32_t iters) {
  // 4 waves x 8 MFMAs per iteration x (32 x 32 x 16 multiply-adds = 32768 FLOP)
  return (double)n_workgroups * 4.0 * 8.0 * (double)iters * 32768.0;
}
