// Routing: group the T*k (token, slot) assignments by expert, stably.
//
// The per-expert sub-batch is the one the paper card ("Outrageously Large
// Neural Networks ... 中文验证版", section 瓶颈) describes: each expert gets the
// rows whose gate kept it.  Positions are expert-contiguous and tokens are
// ascending inside each expert, so the result is unique.
//
// Rank of assignment (t, e) inside expert e = number of earlier tokens that
// kept e.  Tokens are cut into 64-token blocks; inside a block a 64-bit mask
// per expert (bit i = token i of the block kept e) gives the in-block rank by
// a popcount of the bits below the token, and an exclusive scan of the
// per-block counts over the blocks gives the rest.  Every step is integer
// arithmetic, so the result does not depend on scheduling.
//
//   route_hist:    per block, per expert counts  -> blk[b][e]
//   route_colscan: per expert, exclusive scan of blk over b, counts[e]; the
//                  last workgroup to finish scans counts -> offsets
//   route_scatter: pos = offsets[e] + blk[b][e] + in-block rank;
//                  perm[pos] = a, inv[a] = pos
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int SCAN_THREADS = 1024;

// Exclusive scan of n <= 4 * 1024 values held 4 per thread (thread i owns
// v[4i .. 4i+3]); returns the thread's exclusive base and writes the total
// to *total.  Block of 1024 threads.
__device__ int block_scan4(const int v[4], int* total) {
  __shared__ int wsum[SCAN_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int s = v[0] + v[1] + v[2] + v[3];
  int incl = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < SCAN_THREADS / 64; ++i) {
    int x = wsum[i];
    if (i < w) wbase += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - s;
}

__global__ void fill_i32_kernel(int32_t* p, int n, int v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void route_hist_kernel(RouteArgs a) {
  extern __shared__ uint32_t bits[];  // [E][2]
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b == 0 && tid == 0) *a.ticket = 0;
  for (int i = tid; i < 2 * a.E; i += 256) bits[i] = 0u;
  __syncthreads();
  const int64_t t0 = (int64_t)b * ROUTE_BLOCK_TOKENS;
  const int nt = (int)min<int64_t>(ROUTE_BLOCK_TOKENS, a.T - t0);
  for (int i = tid; i < nt * a.k; i += 256) {
    const int tl = i / a.k;
    const int e = a.idx[t0 * a.k + i];
    atomicOr(&bits[2 * e + (tl >> 5)], 1u << (tl & 31));
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += 256)
    a.blk[(int64_t)b * a.E + e] = __popc(bits[2 * e]) + __popc(bits[2 * e + 1]);
}

__global__ __launch_bounds__(SCAN_THREADS) void route_colscan_kernel(RouteArgs a) {
  __shared__ int part[SCAN_THREADS / 64][64];
  __shared__ int last;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int e = blockIdx.x * 64 + lane;
  const int per = (a.NB + 15) / 16;
  const int b0 = w * per, b1 = min(a.NB, b0 + per);
  int s = 0;
  if (e < a.E)
    for (int b = b0; b < b1; ++b) s += a.blk[(int64_t)b * a.E + e];
  part[w][lane] = s;
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < 16; ++i) {
    if (i < w) base += part[i][lane];
    tot += part[i][lane];
  }
  if (e < a.E) {
    int run = base;
    for (int b = b0; b < b1; ++b) {
      int64_t o = (int64_t)b * a.E + e;
      int c = a.blk[o];
      a.blk[o] = run;
      run += c;
    }
    if (w == 0) a.counts[e] = tot;
  }
  // the last workgroup to finish turns counts into offsets
  __threadfence();
  __syncthreads();
  if (tid == 0) last = (atomicAdd(a.ticket, 1) == (int)gridDim.x - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();
  int carry = 0;
  for (int c0 = 0; c0 < a.E; c0 += 4 * SCAN_THREADS) {
    int v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int ee = c0 + 4 * tid + j;
      v[j] = ee < a.E ? __hip_atomic_load(&a.counts[ee], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                      : 0;
    }
    int total;
    int run = carry + block_scan4(v, &total);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int ee = c0 + 4 * tid + j;
      if (ee < a.E) a.offsets[ee] = run;
      run += v[j];
    }
    carry += total;
  }
  if (tid == 0) a.offsets[a.E] = carry;
}

__global__ __launch_bounds__(256) void route_scatter_kernel(RouteArgs a) {
  extern __shared__ uint32_t bits[];  // [E][2]
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < 2 * a.E; i += 256) bits[i] = 0u;
  __syncthreads();
  const int64_t t0 = (int64_t)b * ROUTE_BLOCK_TOKENS;
  const int nt = (int)min<int64_t>(ROUTE_BLOCK_TOKENS, a.T - t0);
  for (int i = tid; i < nt * a.k; i += 256) {
    const int tl = i / a.k;
    const int e = a.idx[t0 * a.k + i];
    atomicOr(&bits[2 * e + (tl >> 5)], 1u << (tl & 31));
  }
  __syncthreads();
  for (int i = tid; i < nt * a.k; i += 256) {
    const int tl = i / a.k;
    const int64_t as = t0 * a.k + i;
    const int e = a.idx[as];
    const uint32_t lo = bits[2 * e], hi = bits[2 * e + 1];
    int below = (tl < 32) ? __popc(lo & ((1u << tl) - 1u))
                          : __popc(lo) + __popc(hi & ((1u << (tl - 32)) - 1u));
    const int pos = a.offsets[e] + a.blk[(int64_t)b * a.E + e] + below;
    a.perm[pos] = (int32_t)as;
    a.inv[as] = pos;
  }
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) {
    // empty batch: counts = 0, offsets = 0
    hipLaunchKernelGGL(fill_i32_kernel, dim3((a.E + 256) / 256), dim3(256), 0, s, a.counts, a.E, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3((a.E + 256) / 256), dim3(256), 0, s, a.offsets,
                       a.E + 1, 0);
    return hipGetLastError();
  }
  size_t sh = sizeof(uint32_t) * 2 * (size_t)a.E;
  hipLaunchKernelGGL(route_hist_kernel, dim3(a.NB), dim3(256), sh, s, a);
  hipLaunchKernelGGL(route_colscan_kernel, dim3((a.E + 63) / 64), dim3(SCAN_THREADS), 0, s, a);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(a.NB), dim3(256), sh, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// tiles[e] = exclusive prefix of ceil(count_e / rows); one workgroup.  With
// desc, tile tiles[e] + i of expert e (count m_e, n_e tiles) covers
// floor(m_e / n_e) rows, plus one for the first m_e % n_e tiles.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(SCAN_THREADS) void tile_map_kernel(const int32_t* offsets, int E,
                                                                int rows, int32_t* tiles,
                                                                int32_t* desc) {
  const int tid = threadIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < E; c0 += 4 * SCAN_THREADS) {
    int v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = c0 + 4 * tid + j;
      v[j] = e < E ? (offsets[e + 1] - offsets[e] + rows - 1) / rows : 0;
    }
    int total;
    int ex = block_scan4(v, &total);
    int run = carry + ex;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = c0 + 4 * tid + j;
      if (e < E) {
        tiles[e] = run;
        if (desc && v[j] > 0) {
          const int m = offsets[e + 1] - offsets[e], base = m / v[j], rem = m % v[j];
          for (int i = 0; i < v[j]; ++i) {
            int32_t* d = desc + 3 * (int64_t)(run + i);
            d[0] = e;
            d[1] = offsets[e] + i * base + min(i, rem);
            d[2] = base + (i < rem ? 1 : 0);
          }
        }
      }
      run += v[j];
    }
    carry += total;
  }
  if (tid == 0) tiles[E] = carry;
}

hipError_t launch_tile_map(const int32_t* offsets, int E, int rows, int32_t* tiles,
                           int32_t* desc, hipStream_t s) {
  hipLaunchKernelGGL(tile_map_kernel, dim3(1), dim3(SCAN_THREADS), 0, s, offsets, E, rows, tiles,
                     desc);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// x_sorted[p] = x[perm[p] / k]; one wave per row, 16-byte chunks when the row
// size allows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* x, const int32_t* perm,
                                                          int k, int64_t A, int64_t row_bytes,
                                                          char* out) {
  const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (p >= A) return;
  const int64_t t = perm[p] / k;
  const char* src = x + t * row_bytes;
  char* dst = out + p * row_bytes;
  if ((row_bytes & 15) == 0) {
    for (int64_t c = lane * 16; c < row_bytes; c += 64 * 16)
      *reinterpret_cast<u32x4*>(dst + c) = *reinterpret_cast<const u32x4*>(src + c);
  } else {
    for (int64_t c = lane; c < row_bytes; c += 64) dst[c] = src[c];
  }
}

hipError_t launch_gather_rows(const void* x, const int32_t* perm, int k, int64_t A, int d,
                              int elem_bytes, void* out, hipStream_t s) {
  if (A == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((A + 3) / 4)), dim3(256), 0, s,
                     (const char*)x, perm, k, A, (int64_t)d * elem_bytes, (char*)out);
  return hipGetLastError();
}

}  // namespace moe
