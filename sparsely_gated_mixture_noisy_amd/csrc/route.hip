// Routing: group the T*k (token, slot) assignments by expert, stably.
//
// The per-expert sub-batch is the one the paper card ("Outrageously Large
// Neural Networks ... 中文验证版", section 瓶颈) describes: each expert gets the
// rows whose gate kept it.  Positions are expert-contiguous and tokens are
// ascending inside each expert, so the result is unique.
//
// Rank of assignment (t, e) inside expert e = number of earlier tokens that
// kept e.  Tokens are cut into 32-token blocks; a 32-bit mask per (block,
// expert) (bit i = token i of the block kept e) gives the in-block rank as a
// popcount of the bits below the token, and an exclusive scan of the mask
// popcounts over the blocks gives the rest.  Every step is integer
// arithmetic, so the result does not depend on scheduling.
//
//   route_hist:    bits[b][e] (the flat gate can write them itself)
//   route_colscan: per expert, exclusive scan of popcount(bits) over b into
//                  base[b][e], and counts[e]
//   route_scatter: every workgroup scans counts into offsets in LDS (cheap,
//                  and no workgroup has to wait for another); workgroup 0
//                  also writes offsets and, when asked, the expert stage's
//                  tile map; pos = offsets[e] + base[b][e] + in-block rank,
//                  perm[pos] = a, inv[a] = pos; with a capacity, ranks at or
//                  past it are dropped (inv[a] = -1) and counts are capped
// With balance partials (per-block gate sums and smooth-load terms from the
// flat gate), route_colscan also reduces them to importance[e] and load[e],
// and workgroup 0 of route_scatter turns those into the CV^2 values.
// No kernel here fences across workgroups: results cross kernel boundaries.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int SCAN_THREADS = 1024;

// Exclusive scan of values held 4 per thread (thread i owns v[4i .. 4i+3]);
// returns the thread's exclusive base and writes the total to *total.
// Block of SCAN_THREADS threads.
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

// Tile map of the expert stage from per-expert row counts: tiles[e] = first
// tile of expert e (exclusive scan of ceil(count / rows)), tiles[E] = total;
// with desc, desc[q] = {expert, first position, rows}, an expert's rows split
// by tile_rows.  counts_of(e) and offsets_of(e) give the routing.
// Called by all SCAN_THREADS threads of one workgroup.
template <typename CountF, typename OffF>
__device__ void build_tile_map(int E, int rows, CountF counts_of, OffF offsets_of, int32_t* tiles,
                               int32_t* desc) {
  const int tid = threadIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < E; c0 += 4 * SCAN_THREADS) {
    int v[4], cnt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = c0 + 4 * tid + j;
      cnt[j] = e < E ? counts_of(e) : 0;
      v[j] = (cnt[j] + rows - 1) / rows;
    }
    int total;
    int run = carry + block_scan4(v, &total);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = c0 + 4 * tid + j;
      if (e < E) {
        tiles[e] = run;
        if (desc && v[j] > 0) {
          const int m = cnt[j], o = offsets_of(e);
          for (int i = 0; i < v[j]; ++i) {
            int32_t* d = desc + 3 * (int64_t)(run + i);
            int first, nr;
            tile_rows(m, v[j], i, &first, &nr);
            d[0] = e;
            d[1] = o + first;
            d[2] = nr;
          }
        }
      }
      run += v[j];
    }
    carry += total;
  }
  if (tid == 0) tiles[E] = carry;
}

__global__ void fill_i32_kernel(int32_t* p, int n, int v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void route_hist_kernel(RouteArgs a) {
  extern __shared__ uint32_t sb[];  // [E]
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int i = tid; i < a.E; i += 256) sb[i] = 0u;
  __syncthreads();
  const int64_t t0 = (int64_t)b * ROUTE_BLOCK_TOKENS;
  const int nt = (int)min<int64_t>(ROUTE_BLOCK_TOKENS, a.T - t0);
  // an index outside [0, E) (caller-supplied) takes no row
  for (int i = tid; i < nt * a.k; i += 256) {
    const int e = a.idx[t0 * a.k + i];
    if ((unsigned)e < (unsigned)a.E) atomicOr(&sb[e], 1u << (i / a.k));
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += 256) a.bits[(int64_t)b * a.E + e] = sb[e];
}

// Workgroup (16 waves) b covers the 16 experts [16b, 16b+16); lane l of wave
// w takes expert 16b + l%16 and the (4w + l/16)-th of 64 contiguous ranges of
// token blocks.  Then wave w scans (counts) and sums (importance, load) the
// 64 range values of expert 16b + w, lane l holding range l.
constexpr int SCAN_EXPERTS = 16;
static_assert(SCAN_THREADS / 64 == SCAN_EXPERTS, "one wave per expert in the range pass");

__global__ __launch_bounds__(SCAN_THREADS) void route_colscan_kernel(RouteArgs a) {
  __shared__ int pc[SCAN_EXPERTS][65];
  __shared__ float pimp[SCAN_EXPERTS][65], pload[SCAN_EXPERTS][65];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int le = lane % SCAN_EXPERTS, range = 4 * w + lane / SCAN_EXPERTS;
  const int e = blockIdx.x * SCAN_EXPERTS + le;
  const int per = (a.NB + 63) / 64;
  const int b0 = range * per, b1 = min(a.NB, b0 + per);
  const bool stats = a.importance != nullptr;
  int s = 0;
  float si = 0.f, sl = 0.f;
  if (e < a.E) {
    // four blocks' loads in flight together; the sums still run in block order
    int b = b0;
    for (; b + 4 <= b1; b += 4) {
      uint32_t wd[4];
      float ip[4], lp[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t o = (int64_t)(b + j) * a.E + e;
        wd[j] = a.bits[o];
        ip[j] = stats ? a.imp_part[o] : 0.f;
        lp[j] = (stats && a.load_part) ? a.load_part[o] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        s += __popc(wd[j]);
        if (stats) {
          si += ip[j];
          if (a.load_part) sl += lp[j];
        }
      }
    }
    for (; b < b1; ++b) {
      const int64_t o = (int64_t)b * a.E + e;
      s += __popc(a.bits[o]);
      if (stats) {
        si += a.imp_part[o];
        if (a.load_part) sl += a.load_part[o];
      }
    }
  }
  pc[le][range] = s;
  pimp[le][range] = si;
  pload[le][range] = sl;
  __syncthreads();
  {
    // importance and load: each range summed in ascending block order above,
    // the 64 range sums by a fixed butterfly here
    const int ew = blockIdx.x * SCAN_EXPERTS + w;
    const int v = pc[w][lane];
    const int incl = wave_incl_scan(v);
    const int tot = __shfl(incl, 63, 64);
    const float ti = wave_sum(pimp[w][lane]);
    const float tl = wave_sum(pload[w][lane]);
    pc[w][lane] = incl - v;  // exclusive base of range `lane` (only wave w touches row w)
    if (lane == 0 && ew < a.E) {
      a.counts[ew] = a.capacity > 0 ? min(tot, a.capacity) : tot;
      if (stats) {
        a.importance[ew] = ti;
        a.load[ew] = a.load_part ? tl : (float)tot;
      }
    }
  }
  __syncthreads();
  if (e < a.E) {
    int run = pc[le][range];
    for (int b = b0; b < b1; ++b) {
      const int64_t o = (int64_t)b * a.E + e;
      a.base[o] = run;
      run += __popc(a.bits[o]);
    }
  }
}

constexpr int SCATTER_THREADS = 256;

// Exclusive scan of counts[0..E) into off[0..E] (LDS) by one workgroup of
// SCATTER_THREADS threads: thread i owns a contiguous run of experts.
__device__ void scan_counts(const int32_t* counts, int E, int* off) {
  const int tid = threadIdx.x;
  const int per = (E + SCATTER_THREADS - 1) / SCATTER_THREADS;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int s = 0;
  for (int e = e0; e < e1; ++e) {
    off[e] = s;
    s += counts[e];
  }
  int total;
  const int base = block_excl_scan<SCATTER_THREADS>(s, &total);
  for (int e = e0; e < e1; ++e) off[e] += base;
  if (tid == 0) off[E] = total;
  __syncthreads();
}

// The expert stage's tile map from the offsets in LDS, by one workgroup of
// SCATTER_THREADS threads: tiles[e] = first tile of expert e (exclusive scan
// of ceil(count / rows)), tiles[E] = total; with desc (may be null),
// desc[q] = {expert, first position, rows}, an expert's rows split by
// tile_rows.
__device__ void scatter_tile_map(const int* off, int E, int rows, int32_t* tiles, int32_t* desc) {
  const int tid = threadIdx.x;
  const int per = (E + SCATTER_THREADS - 1) / SCATTER_THREADS;
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int s = 0;
  for (int e = e0; e < e1; ++e) s += (off[e + 1] - off[e] + rows - 1) / rows;
  int total;
  int run = block_excl_scan<SCATTER_THREADS>(s, &total);
  for (int e = e0; e < e1; ++e) {
    const int m = off[e + 1] - off[e], nt = (m + rows - 1) / rows;
    tiles[e] = run;
    if (desc && nt > 0) {
      for (int i = 0; i < nt; ++i) {
        int32_t* d = desc + 3 * (int64_t)(run + i);
        int first, nr;
        tile_rows(m, nt, i, &first, &nr);
        d[0] = e;
        d[1] = off[e] + first;
        d[2] = nr;
      }
    }
    run += nt;
  }
  if (tid == 0) tiles[E] = total;
}

__global__ __launch_bounds__(SCATTER_THREADS) void route_scatter_kernel(RouteArgs a) {
  extern __shared__ int off[];  // [E+1]
  const int b = blockIdx.x, tid = threadIdx.x;
  scan_counts(a.counts, a.E, off);
  if (b == 0) {
    for (int e = tid; e <= a.E; e += SCATTER_THREADS) a.offsets[e] = off[e];
    if (a.tile_rows > 0) scatter_tile_map(off, a.E, a.tile_rows, a.tiles, a.desc);
    if (a.bal_out) {
      // CV^2 of the vectors the column scan reduced
      const double ci = cv2_of<SCATTER_THREADS>(a.importance, a.E);
      const double cl = cv2_of<SCATTER_THREADS>(a.load, a.E);
      if (tid == 0) {
        a.bal_out[0] = (float)ci;
        a.bal_out[1] = (float)cl;
        a.bal_out[2] = (float)((double)a.w_imp * ci + (double)a.w_load * cl);
      }
    }
  }
  const int64_t t0 = (int64_t)b * ROUTE_BLOCK_TOKENS;
  const int nt = (int)min<int64_t>(ROUTE_BLOCK_TOKENS, a.T - t0);
  for (int i = tid; i < nt * a.k; i += SCATTER_THREADS) {
    const int tl = i / a.k;
    const int64_t as = t0 * a.k + i;
    const int e = a.idx[as];
    if ((unsigned)e >= (unsigned)a.E) {
      a.inv[as] = -1;  // no such expert: the assignment takes no row
      continue;
    }
    const int64_t o = (int64_t)b * a.E + e;
    const int rank = a.base[o] + __popc(a.bits[o] & ((1u << tl) - 1u));
    if (a.capacity > 0 && rank >= a.capacity) {
      a.inv[as] = -1;  // past the expert's capacity: dropped
      continue;
    }
    const int pos = off[e] + rank;
    a.perm[pos] = (int32_t)as;
    a.inv[as] = pos;
  }
  {
    // positions no kept assignment took (a capacity, an index outside
    // [0, E)): a valid index, so that row gathers over all T*k positions stay
    // in bounds; none when every assignment has a row
    const int64_t A = a.T * a.k;
    for (int64_t p = off[a.E] + (int64_t)b * SCATTER_THREADS + tid; p < A;
         p += (int64_t)gridDim.x * SCATTER_THREADS)
      a.perm[p] = 0;
  }
}

// Rows of a keep mask: workgroup b places the tokens of 32-token block b.
// Expert e's kept tokens of the block take ranks base[b][e], +1, ... in
// token order; ranks at or past the cap take no row.
__global__ __launch_bounds__(SCATTER_THREADS) void mask_scatter_kernel(RouteArgs a,
                                                                       int64_t perm_len) {
  extern __shared__ int off[];  // [E+1]
  const int b = blockIdx.x, tid = threadIdx.x;
  scan_counts(a.counts, a.E, off);
  if (b == 0)
    for (int e = tid; e <= a.E; e += SCATTER_THREADS) a.offsets[e] = off[e];
  for (int e = tid; e < a.E; e += SCATTER_THREADS) {
    const int64_t o = (int64_t)b * a.E + e;
    uint32_t rest = a.bits[o];
    int rank = a.base[o];
    while (rest) {
      if (a.capacity > 0 && rank >= a.capacity) break;
      const int i = __ffs(rest) - 1;
      rest &= rest - 1u;
      a.perm[off[e] + rank] = b * ROUTE_BLOCK_TOKENS + i;
      ++rank;
    }
  }
  // rows no kept token took: a valid token, so row gathers stay in bounds
  for (int64_t p = off[a.E] + (int64_t)b * SCATTER_THREADS + tid; p < perm_len;
       p += (int64_t)gridDim.x * SCATTER_THREADS)
    a.perm[p] = 0;
}

hipError_t launch_mask_route(const RouteArgs& a, int64_t perm_len, hipStream_t s) {
  if (a.T == 0) {
    hipLaunchKernelGGL(fill_i32_kernel, dim3((a.E + 256) / 256), dim3(256), 0, s, a.counts, a.E, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3((a.E + 256) / 256), dim3(256), 0, s, a.offsets,
                       a.E + 1, 0);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(route_colscan_kernel, dim3((a.E + SCAN_EXPERTS - 1) / SCAN_EXPERTS),
                     dim3(SCAN_THREADS), 0, s, a);
  hipLaunchKernelGGL(mask_scatter_kernel, dim3(a.NB), dim3(SCATTER_THREADS),
                     sizeof(int) * (size_t)(a.E + 1), s, a, perm_len);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.T == 0) {
    // empty batch: counts = 0, offsets = 0, no tiles
    hipLaunchKernelGGL(fill_i32_kernel, dim3((a.E + 256) / 256), dim3(256), 0, s, a.counts, a.E, 0);
    hipLaunchKernelGGL(fill_i32_kernel, dim3((a.E + 256) / 256), dim3(256), 0, s, a.offsets,
                       a.E + 1, 0);
    if (a.tile_rows > 0)
      hipLaunchKernelGGL(fill_i32_kernel, dim3((a.E + 256) / 256), dim3(256), 0, s, a.tiles,
                         a.E + 1, 0);
    return hipGetLastError();
  }
  if (!a.have_bits)
    hipLaunchKernelGGL(route_hist_kernel, dim3(a.NB), dim3(256), sizeof(uint32_t) * (size_t)a.E, s,
                       a);
  hipLaunchKernelGGL(route_colscan_kernel, dim3((a.E + SCAN_EXPERTS - 1) / SCAN_EXPERTS),
                     dim3(SCAN_THREADS), 0, s, a);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(a.NB), dim3(SCATTER_THREADS),
                     sizeof(int) * (size_t)(a.E + 1), s, a);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int n, int v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Stand-alone tile map (one workgroup) for the expert stage called on its own.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(SCAN_THREADS) void tile_map_kernel(const int32_t* offsets, int E,
                                                                int rows, int32_t* tiles,
                                                                int32_t* desc) {
  build_tile_map(
      E, rows, [&](int e) { return offsets[e + 1] - offsets[e]; },
      [&](int e) { return offsets[e]; }, tiles, desc);
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
