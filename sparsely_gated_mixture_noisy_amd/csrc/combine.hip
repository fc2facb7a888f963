// Combine and balance statistics.
//
// Combine ("MoE:稀疏门控混合专家", nengyongai.cn, section 二):
//   y_t = sum over the token's kept slots s (ascending) of
//         gate[t][s] * y_sorted[inv[t*k + s]],  fp32 accumulation.
// One wave per token; each lane owns 16-byte column chunks of the row.
//
// Balance statistics ("Outrageously Large Neural Networks — MoE ..." reading
// note, sections 核心想法 and 方法怎么做; paper card, section 方法适配):
//   importance[e] = sum of the gates routed to e, summed over e's routed
//                   positions by one wave (lane-strided partial sums, then a
//                   fixed shuffle tree);
//   load[e]       = fixed-order sum of per-workgroup partials of the smooth
//                   load, or the row count when there is no noise;
//   CV^2          = population variance / mean^2, reduced in fp64.
// No floating-point atomics anywhere: results are bitwise reproducible.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ ys,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ gate, int64_t Tn,
                                                      int k, int d, T* __restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= Tn) return;
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte chunk
  int rows[8];
  float g[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    rows[s] = s < k ? inv[t * k + s] : 0;
    g[s] = s < k ? gate[t * k + s] : 0.f;
  }
  if (d % V == 0) {
    for (int c = lane * V; c < d; c += 64 * V) {
      float acc[V];
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s < k) {
          const T* src = ys + (int64_t)rows[s] * d + c;
          u32x4 raw = *reinterpret_cast<const u32x4*>(src);
          const T* vals = reinterpret_cast<const T*>(&raw);
#pragma unroll
          for (int j = 0; j < V; ++j) acc[j] = fmaf(g[s], Elem<T>::load(vals, j), acc[j]);
        }
      }
      u32x4 out;
      T* ov = reinterpret_cast<T*>(&out);
#pragma unroll
      for (int j = 0; j < V; ++j) Elem<T>::store(ov, j, acc[j]);
      *reinterpret_cast<u32x4*>(y + t * d + c) = out;
    }
  } else {
    for (int c = lane; c < d; c += 64) {
      float acc = 0.f;
      for (int s = 0; s < k; ++s) acc = fmaf(g[s], Elem<T>::load(ys, (int64_t)rows[s] * d + c), acc);
      Elem<T>::store(y, t * d + c, acc);
    }
  }
}

hipError_t launch_combine(const void* y_sorted, const int32_t* inv, const float* gate, int64_t T,
                          int k, int d, bool bf16, void* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  dim3 grid((unsigned)((T + 3) / 4));
  if (bf16)
    hipLaunchKernelGGL(combine_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)y_sorted, inv,
                       gate, T, k, d, (bf16_t*)y);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s, (const float*)y_sorted, inv,
                       gate, T, k, d, (float*)y);
  return hipGetLastError();
}

// One wave per expert: importance[e] = sum_{p in segment e} gate[perm[p]].
__global__ __launch_bounds__(256) void importance_kernel(const int32_t* perm,
                                                        const int32_t* offsets,
                                                        const float* gate, int E,
                                                        float* importance) {
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= E) return;
  const int p0 = offsets[e], p1 = offsets[e + 1];
  float s = 0.f;
  for (int p = p0 + lane; p < p1; p += 64) s += gate[perm[p]];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) importance[e] = s;
}

hipError_t launch_importance(const int32_t* perm, const int32_t* offsets, const float* gate,
                             int E, float* importance, hipStream_t s) {
  hipLaunchKernelGGL(importance_kernel, dim3((E + 3) / 4), dim3(256), 0, s, perm, offsets, gate, E,
                     importance);
  return hipGetLastError();
}

// load[e] = sum_b part[b][e] in a fixed order, or the row count of e.
// Workgroup: 64 experts x 16 waves; wave w sums a contiguous range of b in
// ascending order, then the 16 wave sums are added in wave order.
__global__ __launch_bounds__(1024) void load_reduce_kernel(const float* part, int blocks,
                                                          const int32_t* offsets, int E,
                                                          float* load) {
  __shared__ float red[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  if (!part) {
    if (w == 0 && e < E) load[e] = (float)(offsets[e + 1] - offsets[e]);
    return;
  }
  const int per = (blocks + 15) / 16;
  const int b0 = w * per, b1 = min(blocks, b0 + per);
  float s = 0.f;
  if (e < E)
    for (int b = b0; b < b1; ++b) s += part[(int64_t)b * E + e];
  red[w][lane] = s;
  __syncthreads();
  if (w == 0 && e < E) {
    float t = 0.f;
    for (int i = 0; i < 16; ++i) t += red[i][lane];
    load[e] = t;
  }
}

hipError_t launch_load_reduce(const float* part, int blocks, const int32_t* offsets, int E,
                              float* load, hipStream_t s) {
  hipLaunchKernelGGL(load_reduce_kernel, dim3((E + 63) / 64), dim3(1024), 0, s, part, blocks,
                     offsets, E, load);
  return hipGetLastError();
}

// Fixed-order fp64 block reduction (256 threads).
__device__ double block_sum_f64(double v) {
  __shared__ double red[256];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  double r = red[0];
  __syncthreads();
  return r;
}

__device__ double cv2_of(const float* v, int E) {
  double s = 0.0;
  for (int i = threadIdx.x; i < E; i += 256) s += (double)v[i];
  const double mean = block_sum_f64(s) / E;
  double q = 0.0;
  for (int i = threadIdx.x; i < E; i += 256) {
    double dv = (double)v[i] - mean;
    q += dv * dv;
  }
  const double var = block_sum_f64(q) / E;
  return mean == 0.0 ? 0.0 : var / (mean * mean);
}

__global__ __launch_bounds__(256) void cv2_kernel(const float* importance, const float* load,
                                                 int E, float w_imp, float w_load, float* out) {
  const double ci = cv2_of(importance, E);
  const double cl = cv2_of(load, E);
  if (threadIdx.x == 0) {
    out[0] = (float)ci;
    out[1] = (float)cl;
    out[2] = (float)((double)w_imp * ci + (double)w_load * cl);
  }
}

hipError_t launch_cv2(const float* importance, const float* load, int E, float w_imp,
                      float w_load, float* out, hipStream_t s) {
  hipLaunchKernelGGL(cv2_kernel, dim3(1), dim3(256), 0, s, importance, load, E, w_imp, w_load, out);
  return hipGetLastError();
}

}  // namespace moe
