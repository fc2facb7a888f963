// The generator's noise written out as tensors (moe_draw_noise): the same
// draws the gate kernels take when they generate the noise themselves.
#include "moe_kernels.h"

namespace moe {

// eps[t][g][j] (G groups of n; the flat noise is G = 1) of one stream
__global__ __launch_bounds__(256) void draw_noise_kernel(int64_t T, int G, int n, int stream,
                                                         uint32_t k0, uint32_t k1, float* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * G * n) return;
  const int j = (int)(i % n);
  const int64_t r = i / n;
  const int g = (int)(r % G);
  const int64_t t = r / G;
  out[i] = noise_normal((uint32_t)j, (uint32_t)t, (uint32_t)g, (uint32_t)stream, k0, k1);
}

hipError_t launch_draw_noise(int64_t T, int E, int G, uint64_t seed, float* eps, float* eps_p,
                             hipStream_t s) {
  const uint32_t k0 = (uint32_t)(seed & 0xFFFFFFFFu), k1 = (uint32_t)(seed >> 32);
  const int groups = G > 0 ? G : 1, n = E / groups;
  if (eps && T > 0) {
    const int64_t total = T * groups * n;
    hipLaunchKernelGGL(draw_noise_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       T, groups, n, 0, k0, k1, eps);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (eps_p && G > 0 && T > 0) {
    const int64_t total = T * G;
    hipLaunchKernelGGL(draw_noise_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       T, 1, G, 1, k0, k1, eps_p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace moe
