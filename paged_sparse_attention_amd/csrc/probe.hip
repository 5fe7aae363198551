// probe.hip -- measurement helper: sustained bf16 MFMA rate of the part.
//
// Not a step of the attention path.  The benchmark divides the attention
// kernels' credited flops by the published bf16 peak and also by the rate this
// kernel reaches, so that the fraction can be read against what the matrix
// cores deliver on the box.  Each wave keeps four independent 32x32x16
// accumulation chains in registers (no memory traffic inside the loop) and
// issues 4 * iters MFMAs of 32768 flop each.
#include "common.h"

namespace oomb {

constexpr int kProbeWaves = 4;
constexpr int kProbeChains = 4;

__global__ __launch_bounds__(kProbeWaves * 64) void mfma_probe_kernel(int iters, float* out) {
  // A = 1/16 everywhere, B = 1 everywhere: every MFMA adds 16 * (1/16) = 1 to
  // each accumulator element, exactly, so each element ends at iters.
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)0.0625f;
    b[i] = (__bf16)1.0f;
  }
  f32x16 c[kProbeChains];
#pragma unroll
  for (int k = 0; k < kProbeChains; ++k) c[k] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kProbeChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kProbeChains; ++k) s += c[k][threadIdx.x & 15];
  if ((threadIdx.x & 63) == 0) out[blockIdx.x * kProbeWaves + (threadIdx.x >> 6)] = s;
}

hipError_t launch_probe_mfma(int n_blocks, int iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_blocks), dim3(kProbeWaves * 64), 0, st, iters, out);
  return hipGetLastError();
}

}  // namespace oomb
