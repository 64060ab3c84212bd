// Gradient of the attention sinks: one logit sigma_h per query head joins
// every row's softmax normalizer as an extra score whose value row is zero,
// so its probability is p_i = exp(sigma_h - lse_i) and the chain rule through
// that column gives d sigma_h = -sum over batches and rows of p_i * Delta_i,
// Delta_i = <dO_i, O_i> (page "Lab 028 lab detail: Off NVIDIA, you fix the
// platform yourself", "What I changed, in plain terms", item 2, lists sinks
// among the backward's parameters). Both inputs are one float per query row,
// already in memory after the dQ pass: this is a small reduction, one
// workgroup per head, in a fixed order (bitwise reproducible).
#include <math.h>

#include "common.h"

namespace sdpa {

__global__ void __launch_bounds__(256)
dsinks_kernel(const float* __restrict__ LSE, const float* __restrict__ Delta, const float* __restrict__ Sinks,
              float* __restrict__ dSinks, int B, int Hq, int Lq) {
  __shared__ float part[256];
  const int h = blockIdx.x, tid = threadIdx.x;
  const float sg = Sinks[h];
  float acc = 0.f;
  if (sg != -INFINITY) {
    for (int b = 0; b < B; b++) {
      const size_t row0 = ((size_t)b * Hq + h) * Lq;
      for (int i = tid; i < Lq; i += 256) acc += expf(sg - LSE[row0 + i]) * Delta[row0 + i];
    }
  }
  part[tid] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (tid < s) part[tid] += part[tid + s];
    __syncthreads();
  }
  if (tid == 0) dSinks[h] = -part[0];
}

hipError_t launch_dsinks(const float* lse, const float* delta, const float* sinks, float* dsinks, int B, int Hq,
                         int Lq, hipStream_t stream) {
  if (Hq == 0) return hipSuccess;
  hipLaunchKernelGGL(dsinks_kernel, dim3((unsigned)Hq), dim3(256), 0, stream, lse, delta, sinks, dsinks, B, Hq, Lq);
  return hipGetLastError();
}

}  // namespace sdpa
