// Combine and balance statistics.
//
// Combine ("MoE:稀疏门控混合专家", nengyongai.cn, section 二):
//   y_t = sum over the token's kept slots s (ascending) of
//         gate[t][s] * y_sorted[inv[t*k + s]],  fp32 accumulation;
//   slots that an expert's capacity dropped (inv = -1) add nothing.
// One wave per token; each lane owns 16-byte column chunks of the row.
//
// Balance statistics ("Outrageously Large Neural Networks — MoE ..." reading
// note, sections 核心想法 and 方法怎么做; paper card, section 方法适配):
//   importance[e] = sum of the gates routed to e;
//   load[e]       = sum of the smooth-load terms of e, or its row count when
//                   there is no noise;
//   CV^2          = population variance / mean^2, reduced in fp64.
// No floating-point atomics anywhere: results are bitwise reproducible.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

// K (the slots per token) is a template argument, so that every slot's row
// load is issued before the first one is used; a dropped slot reads row 0
// and adds nothing.
template <typename T, int K>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ ys,
                                                      const int32_t* __restrict__ inv,
                                                      const float* __restrict__ gate, int64_t Tn,
                                                      int d, T* __restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= Tn) return;
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte chunk
  int rows[K];
  float g[K];
#pragma unroll
  for (int s = 0; s < K; ++s) {
    rows[s] = inv[t * K + s];
    g[s] = gate[t * K + s];
  }
  if (d % V == 0) {
    for (int c = lane * V; c < d; c += 64 * V) {
      u32x4 raw[K];
#pragma unroll
      for (int s = 0; s < K; ++s)
        raw[s] = *reinterpret_cast<const u32x4*>(ys + (int64_t)max(rows[s], 0) * d + c);
      float acc[V];
#pragma unroll
      for (int j = 0; j < V; ++j) acc[j] = 0.f;
#pragma unroll
      for (int s = 0; s < K; ++s) {
        const T* vals = reinterpret_cast<const T*>(&raw[s]);
        const bool keep = rows[s] >= 0;
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const float f = fmaf(g[s], Elem<T>::load(vals, j), acc[j]);
          acc[j] = keep ? f : acc[j];
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
#pragma unroll
      for (int s = 0; s < K; ++s)
        if (rows[s] >= 0) acc = fmaf(g[s], Elem<T>::load(ys, (int64_t)rows[s] * d + c), acc);
      Elem<T>::store(y, t * d + c, acc);
    }
  }
}

template <typename T, int K>
static hipError_t launch_combine_k(const void* y_sorted, const int32_t* inv, const float* gate,
                                   int64_t T_, int d, void* y, hipStream_t s) {
  hipLaunchKernelGGL((combine_kernel<T, K>), dim3((unsigned)((T_ + 3) / 4)), dim3(256), 0, s,
                     (const T*)y_sorted, inv, gate, T_, d, (T*)y);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_combine_t(const void* y_sorted, const int32_t* inv, const float* gate,
                                   int64_t T_, int k, int d, void* y, hipStream_t s) {
  switch (k) {
    case 1: return launch_combine_k<T, 1>(y_sorted, inv, gate, T_, d, y, s);
    case 2: return launch_combine_k<T, 2>(y_sorted, inv, gate, T_, d, y, s);
    case 3: return launch_combine_k<T, 3>(y_sorted, inv, gate, T_, d, y, s);
    case 4: return launch_combine_k<T, 4>(y_sorted, inv, gate, T_, d, y, s);
    case 5: return launch_combine_k<T, 5>(y_sorted, inv, gate, T_, d, y, s);
    case 6: return launch_combine_k<T, 6>(y_sorted, inv, gate, T_, d, y, s);
    case 7: return launch_combine_k<T, 7>(y_sorted, inv, gate, T_, d, y, s);
    case 8: return launch_combine_k<T, 8>(y_sorted, inv, gate, T_, d, y, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_combine(const void* y_sorted, const int32_t* inv, const float* gate, int64_t T,
                          int k, int d, bool bf16, void* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  return bf16 ? launch_combine_t<bf16_t>(y_sorted, inv, gate, T, k, d, y, s)
              : launch_combine_t<float>(y_sorted, inv, gate, T, k, d, y, s);
}

// ---------------------------------------------------------------------------
// Balance statistics in one launch.  Workgroup (16 waves) b covers the 16
// experts [16b, 16b+16).  Both sums run over 64 contiguous ranges of 32-token
// blocks: each range is summed in ascending block order, then the 64 range
// sums by a fixed butterfly (the same order in which the routing step reduces
// the flat gate's per-block partials, so both give the same bits):
//   importance[e]: wave w takes expert 16b + w, lane l range l, the block
//                  sums adding the block's gates in token order;
//   load[e]:       lane l of wave w takes expert 16b + l%16 and range
//                  4w + l/16 of the load-partial rows (or the row count
//                  without partials).
// A one-workgroup kernel then reduces both vectors to CV^2 in fp64 with a
// fixed tree.
// ---------------------------------------------------------------------------
constexpr int BAL_THREADS = 1024;
constexpr int BAL_EXPERTS = 16;

__global__ __launch_bounds__(BAL_THREADS) void balance_kernel(BalanceArgs a) {
  __shared__ float red[BAL_EXPERTS][65];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e0 = blockIdx.x * BAL_EXPERTS;
  const int per = (a.blocks + 63) / 64;
  {
    // load partials: lane l of wave w sums range 4w + l/16 of expert 16b + l%16
    const int le = lane % BAL_EXPERTS, range = 4 * w + lane / BAL_EXPERTS;
    const int e = e0 + le;
    float s = 0.f;
    if (a.part && e < a.E) {
      const int b0 = range * per, b1 = min(a.blocks, b0 + per);
      for (int b = b0; b < b1; ++b) s += a.part[(int64_t)b * a.E + e];
    }
    red[le][range] = s;
  }
  // importance of expert e0 + w; lane l sums the 32-token blocks
  // [l*per, (l+1)*per): e's positions are in ascending token order, so the
  // lane binary-searches its first one and walks on, adding each block's
  // gates in row order into a block sum and the block sums in order
  const int e = e0 + w;
  float rs = 0.f;
  if (e < a.E) {
    const int p0 = a.offsets[e], p1 = a.offsets[e + 1];
    const int64_t tb0 = (int64_t)lane * per * 32, tb1 = tb0 + (int64_t)per * 32;
    int lo = p0, hi = p1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (a.perm[mid] / a.k < tb0) lo = mid + 1; else hi = mid;
    }
    float bs = 0.f;
    int64_t cur = -1;
    for (int q = lo; q < p1; ++q) {
      const int as = a.perm[q];
      const int64_t t = as / a.k;
      if (t >= tb1) break;
      if (t / 32 != cur) {
        if (cur >= 0) rs += bs;
        bs = 0.f;
        cur = t / 32;
      }
      bs += a.gate[as];
    }
    if (cur >= 0) rs += bs;
  }
  __syncthreads();
  // the 64 range sums of expert e0 + w by the same butterfly as the routing
  // step's reduction
  const float ti = wave_sum(rs);
  const float tl = wave_sum(red[w][lane]);
  if (lane == 0 && e < a.E) {
    a.importance[e] = ti;
    a.load[e] = a.part ? tl : (float)(a.offsets[e + 1] - a.offsets[e]);
  }
}

__global__ __launch_bounds__(BAL_THREADS) void cv2_kernel(BalanceArgs a) {
  const double ci = cv2_of<BAL_THREADS>(a.importance, a.E);
  const double cl = cv2_of<BAL_THREADS>(a.load, a.E);
  if (threadIdx.x == 0) {
    a.out[0] = (float)ci;
    a.out[1] = (float)cl;
    a.out[2] = (float)((double)a.w_imp * ci + (double)a.w_load * cl);
  }
}

hipError_t launch_cv2(const float* importance, const float* load, int E, float w_imp,
                      float w_load, float* out, hipStream_t s) {
  BalanceArgs a{};
  a.importance = const_cast<float*>(importance);
  a.load = const_cast<float*>(load);
  a.E = E;
  a.w_imp = w_imp;
  a.w_load = w_load;
  a.out = out;
  hipLaunchKernelGGL(cv2_kernel, dim3(1), dim3(BAL_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_balance(const BalanceArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(balance_kernel, dim3((a.E + BAL_EXPERTS - 1) / BAL_EXPERTS),
                     dim3(BAL_THREADS), 0, s, a);
  hipLaunchKernelGGL(cv2_kernel, dim3(1), dim3(BAL_THREADS), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
