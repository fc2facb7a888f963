// Gate kernels: noisy scores, KeepTopK, softmax over the kept scores, and the
// smooth load estimate.
//
// Method ("MoE:稀疏门控混合专家", nengyongai.cn, sections 三 and 四):
//   clean_e = x . W_g[e] (+ bias_e)
//   H_e     = clean_e + eps_e * softplus(x . W_noise[e])   (noisy gate)
//   keep the k largest H_e (ties: lower e), softmax over the kept ones.
//
// One workgroup scores a tile of 32 rows against all experts, 128 projection
// columns at a time (64 experts x {clean, raw} when noisy, 128 experts
// otherwise).  bf16 projections run on v_mfma_f32_32x32x16_bf16 straight from
// global memory (each wave owns one 32-column block); the per-row top-(k+1)
// lists live in registers, 8 lanes per row, and are merged with lane shuffles.
#include "moe_device.h"
#include "moe_kernels.h"

#include <algorithm>

namespace moe {

constexpr int GATE_ROWS = 32;
constexpr int GATE_THREADS = 256;
typedef float ProjTile[GATE_ROWS][GATE_ROWS + 1];

// One projection chunk is 4 column blocks of 32 columns.  Block b computes
// P[b][r][c] = x[rows[r]] . tab[row0 + c] for c < valid; columns at or past
// `valid` read table row `safe` and are never used.  Columns of chunk cb:
// noisy -> blocks 0,1 clean scores of experts cb..cb+63, blocks 2,3 the raw
// noise scores of the same experts; noise-free -> blocks 0..3 clean scores of
// experts cb..cb+127.  Expert e is table row tab_row0 + e.
struct BlockCols {
  const void* tab;
  int row0, valid, safe;
};

__device__ __forceinline__ BlockCols block_cols(int b, const void* wg, const void* wn, bool noisy,
                                                int tab_row0, int cb, int nvalid) {
  BlockCols bc;
  const int e0 = noisy ? (b & 1) * 32 : b * 32;
  bc.tab = (noisy && b >= 2) ? wn : wg;
  bc.row0 = tab_row0 + cb + e0;
  bc.valid = max(0, min(32, nvalid - e0));
  bc.safe = tab_row0;
  return bc;
}

struct ChunkSpec {
  const void* wg;
  const void* wn;
  bool noisy;
  int tab_row0, cb, nvalid;
};

template <typename T>
struct Proj;

template <>
struct Proj<bf16_t> {
  static __device__ __forceinline__ void run(const bf16_t* __restrict__ x, int d, const int* rows,
                                             const ChunkSpec& cs, ProjTile* P) {
    const int lane = threadIdx.x & 63, b = threadIdx.x >> 6;
    const int c = lane & 31, kh = (lane >> 5) * 8;
    const BlockCols bc = block_cols(b, cs.wg, cs.wn, cs.noisy, cs.tab_row0, cs.cb, cs.nvalid);
    const int trow = c < bc.valid ? bc.row0 + c : bc.safe;
    const bf16_t* wp = (const bf16_t*)bc.tab + (int64_t)trow * d + kh;
    const bf16_t* xp = x + (int64_t)rows[c] * d + kh;
    f32x16 acc = {};
    int k0 = 0;
    for (; k0 + 64 <= d; k0 += 64) {
      bf16x8 a0 = load_bf16x8(xp + k0), b0 = load_bf16x8(wp + k0);
      bf16x8 a1 = load_bf16x8(xp + k0 + 16), b1 = load_bf16x8(wp + k0 + 16);
      bf16x8 a2 = load_bf16x8(xp + k0 + 32), b2 = load_bf16x8(wp + k0 + 32);
      bf16x8 a3 = load_bf16x8(xp + k0 + 48), b3 = load_bf16x8(wp + k0 + 48);
      acc = mfma32(a0, b0, acc);
      acc = mfma32(a1, b1, acc);
      acc = mfma32(a2, b2, acc);
      acc = mfma32(a3, b3, acc);
    }
    for (; k0 < d; k0 += 16) acc = mfma32(load_bf16x8(xp + k0), load_bf16x8(wp + k0), acc);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      int r = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
      P[b][r][c] = acc[i];
    }
  }
};

template <>
struct Proj<float> {
  static __device__ __forceinline__ void run(const float* __restrict__ x, int d, const int* rows,
                                             const ChunkSpec& cs, ProjTile* P) {
    const int col = threadIdx.x & 127;
    const int b = col >> 5, c = col & 31;
    const BlockCols bc = block_cols(b, cs.wg, cs.wn, cs.noisy, cs.tab_row0, cs.cb, cs.nvalid);
    const int trow = c < bc.valid ? bc.row0 + c : bc.safe;
    const float* wp = (const float*)bc.tab + (int64_t)trow * d;
    for (int r = threadIdx.x >> 7; r < GATE_ROWS; r += 2) {
      const float* xp = x + (int64_t)rows[r] * d;
      float s = 0.f;
      for (int k = 0; k < d; ++k) s = fmaf(xp[k], wp[k], s);
      P[b][r][c] = s;
    }
  }
};

// Running top-K1 list of one lane (best first).
template <int K1>
struct TopList {
  float v[K1];
  int e[K1];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < K1; ++j) { v[j] = -INFINITY; e[j] = 0x7fffffff; }
  }
  __device__ __forceinline__ void insert(float cv, int ce) {
    if (!ranks_before(cv, ce, v[K1 - 1], e[K1 - 1])) return;
    v[K1 - 1] = cv;
    e[K1 - 1] = ce;
#pragma unroll
    for (int j = K1 - 1; j > 0; --j) {
      if (ranks_before(v[j], e[j], v[j - 1], e[j - 1])) {
        float tv = v[j]; v[j] = v[j - 1]; v[j - 1] = tv;
        int te = e[j]; e[j] = e[j - 1]; e[j - 1] = te;
      }
    }
  }
  // Merge the lists of the 8 lanes of a row group: every lane ends with the
  // group's best K1 (value, expert) pairs in rank order.
  __device__ __forceinline__ void merge8(float* ov, int* oe) {
#pragma unroll
    for (int round = 0; round < K1; ++round) {
      float bv = v[0];
      int be = e[0];
#pragma unroll
      for (int off = 1; off < 8; off <<= 1) {
        float v2 = __shfl_xor(bv, off, 8);
        int e2 = __shfl_xor(be, off, 8);
        if (ranks_before(v2, e2, bv, be)) { bv = v2; be = e2; }
      }
      ov[round] = bv;
      oe[round] = be;
      if (e[0] == be) {
#pragma unroll
        for (int j = 0; j < K1 - 1; ++j) { v[j] = v[j + 1]; e[j] = e[j + 1]; }
        v[K1 - 1] = -INFINITY;
        e[K1 - 1] = 0x7fffffff;
      }
    }
  }
};

// Scores of one 32-row tile against experts [0, E) of a table block, merged
// into per-lane top-K1 lists.  Table row of expert e is tab_row0 + e; the
// noise draw of (tile row r, expert e) is erow[e] with erow the row's eps
// pointer (unused when !noisy).
template <typename T, int K1>
__device__ void score_tile(const T* __restrict__ x, int d, const int* rows, const void* wg,
                           const void* wn, const float* __restrict__ bias, int tab_row0, int E,
                           const float* erow, bool noisy, ProjTile* P, TopList<K1>& L) {
  const int tid = threadIdx.x;
  const int row = tid >> 3, sub = tid & 7;
  const int ce = noisy ? 64 : 128;  // experts per chunk
  for (int cb = 0; cb < E; cb += ce) {
    const int nvalid = min(ce, E - cb);
    const ChunkSpec cs{wg, wn, noisy, tab_row0, cb, nvalid};
    __syncthreads();  // P is free
    Proj<T>::run(x, d, rows, cs, P);
    __syncthreads();
    for (int j = sub; j < nvalid; j += 8) {
      const int e = cb + j;
      float c = P[j >> 5][row][j & 31];
      if (bias) c += bias[tab_row0 + e];
      float h = c;
      if (noisy) {
        float raw = P[2 + (j >> 5)][row][j & 31];
        h = c + erow[e] * softplus_f(raw);
      }
      L.insert(h, e);
    }
  }
}

// Turn the merged top-(k+1) of a row (rank order) into the kept experts in
// ascending index order and their softmax gates; also the k-th and (k+1)-th
// scores.  Valid in every lane; entries >= k are padding.
template <int K1>
__device__ __forceinline__ void kept_gates(const float* ov, const int* oe, int k, int E,
                                           int* ke, float* kg, float* kth, float* k1th) {
  float kv[K1];
#pragma unroll
  for (int j = 0; j < K1; ++j) {
    ke[j] = j < k ? oe[j] : 0x7fffffff;
    kv[j] = ov[j];
  }
  // ascending expert order over the first k entries (padding sorts last)
#pragma unroll
  for (int i = 1; i < K1; ++i) {
#pragma unroll
    for (int j = K1 - 1; j >= i; --j) {
      if (ke[j] < ke[j - 1]) {
        int te = ke[j]; ke[j] = ke[j - 1]; ke[j - 1] = te;
        float tv = kv[j]; kv[j] = kv[j - 1]; kv[j - 1] = tv;
      }
    }
  }
  const float m = ov[0];
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < K1; ++j) {
    float w = j < k ? expf(kv[j] - m) : 0.f;
    kg[j] = w;
    s += w;
  }
  const float inv = 1.0f / s;
#pragma unroll
  for (int j = 0; j < K1; ++j) kg[j] *= inv;
  float a = ov[0], b = -INFINITY;
#pragma unroll
  for (int j = 0; j < K1; ++j) {
    if (j == k - 1) a = ov[j];
    if (j == k) b = ov[j];
  }
  *kth = a;
  *k1th = (k < E) ? b : -INFINITY;
}

// ---------------------------------------------------------------------------
// Flat gate: tile = 32 consecutive tokens.
// ---------------------------------------------------------------------------
template <typename T, int K1>
__global__ __launch_bounds__(GATE_THREADS) void gate_flat_kernel(GateFlatArgs a) {
  __shared__ ProjTile P[4];
  __shared__ int rows[GATE_ROWS];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * GATE_ROWS;
  if (tid < GATE_ROWS) rows[tid] = (int)min<int64_t>(t0 + tid, a.T - 1);
  __syncthreads();
  const int row = tid >> 3;
  const int64_t t = t0 + row;
  const float* erow = a.eps ? a.eps + (int64_t)rows[row] * a.E : nullptr;
  TopList<K1> L;
  L.init();
  score_tile<T, K1>((const T*)a.x, a.d, rows, a.w_gate, a.w_noise, a.bias, 0, a.E, erow,
                    a.eps != nullptr && a.w_noise != nullptr, P, L);
  float ov[K1];
  int oe[K1];
  L.merge8(ov, oe);
  if ((tid & 7) == 0 && t < a.T) {
    int ke[K1];
    float kg[K1], kth, k1th;
    kept_gates<K1>(ov, oe, a.k, a.E, ke, kg, &kth, &k1th);
#pragma unroll
    for (int j = 0; j < K1; ++j) {
      if (j < a.k) {
        a.idx[t * a.k + j] = ke[j];
        a.gate[t * a.k + j] = kg[j];
      }
    }
    if (a.thr) {
      a.thr[2 * t] = kth;
      a.thr[2 * t + 1] = k1th;
    }
  }
}

// ---------------------------------------------------------------------------
// Secondary gate of the hierarchy: rows are the (token, kept group) pairs of
// one group g, taken from the group routing (perm_g, offsets_g); tile i of
// group g covers positions offsets_g[g] + 32*(i - tiles_g[g]) onward.
// Writes the final experts g*Eg + j and gates gate_p * gate_s directly.
// ---------------------------------------------------------------------------
template <typename T, int K1>
__global__ __launch_bounds__(GATE_THREADS) void gate_group_kernel(GateGroupArgs a) {
  __shared__ ProjTile P[4];
  __shared__ int rows[GATE_ROWS];
  __shared__ int asg[GATE_ROWS];
  __shared__ int s_g, s_p0, s_n;
  const int tid = threadIdx.x;
  if (tid == 0) {
    int q = blockIdx.x, g = -1;
    for (int i = 0; i < a.G; ++i)
      if (q >= a.tiles_g[i] && q < a.tiles_g[i + 1]) g = i;
    s_g = g;
    if (g >= 0) {
      int p0 = a.offsets_g[g] + GATE_ROWS * (q - a.tiles_g[g]);
      s_p0 = p0;
      s_n = min(GATE_ROWS, a.offsets_g[g + 1] - p0);
    }
  }
  __syncthreads();
  const int g = s_g;
  if (g < 0) return;
  const int p0 = s_p0, n = s_n;
  if (tid < GATE_ROWS) {
    int as = a.perm_g[p0 + min(tid, n - 1)];
    asg[tid] = as;
    rows[tid] = as / a.kg;
  }
  __syncthreads();
  const int row = tid >> 3;
  const int Eg = a.Eg;
  const float* erow = a.eps ? a.eps + ((int64_t)rows[row] * a.G + g) * Eg : nullptr;
  TopList<K1> L;
  L.init();
  score_tile<T, K1>((const T*)a.x, a.d, rows, a.w_gate, a.w_noise, nullptr, g * Eg, Eg, erow,
                    a.eps != nullptr && a.w_noise != nullptr, P, L);
  float ov[K1];
  int oe[K1];
  L.merge8(ov, oe);
  if ((tid & 7) == 0 && row < n) {
    int ke[K1];
    float kg[K1], kth, k1th;
    kept_gates<K1>(ov, oe, a.kpg, Eg, ke, kg, &kth, &k1th);
    const int as = asg[row];
    const int64_t t = as / a.kg;
    const int sg = as % a.kg;
    const float gp = a.gate_p[as];
    const int k = a.kg * a.kpg;
#pragma unroll
    for (int j = 0; j < K1; ++j) {
      if (j < a.kpg) {
        a.idx[t * k + sg * a.kpg + j] = g * Eg + ke[j];
        a.gate[t * k + sg * a.kpg + j] = gp * kg[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Smooth load estimate (flat noisy gate).  Each workgroup covers `tiles`
// consecutive 32-token tiles and accumulates, per expert e,
//   sum_t Phi((clean[t,e] - theta[t,e]) / softplus(raw[t,e]))
// with theta = thr[t][1] if e is kept by t, else thr[t][0].  The per-expert
// partial sums of the workgroup go to part[blockIdx.x][E] (summed over rows
// in ascending order), reduced across workgroups in a fixed order later.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(GATE_THREADS) void load_partial_kernel(LoadArgs a) {
  __shared__ ProjTile P[4];
  __shared__ int rows[GATE_ROWS];
  __shared__ float Q[GATE_ROWS][65];
  extern __shared__ float acc[];  // [E]
  const int tid = threadIdx.x;
  const int row = tid >> 3, sub = tid & 7;
  for (int e = tid; e < a.E; e += GATE_THREADS) acc[e] = 0.f;
  for (int tt = 0; tt < a.tiles; ++tt) {
    const int64_t t0 = ((int64_t)blockIdx.x * a.tiles + tt) * GATE_ROWS;
    if (t0 >= a.T) break;
    __syncthreads();
    if (tid < GATE_ROWS) rows[tid] = (int)min<int64_t>(t0 + tid, a.T - 1);
    __syncthreads();
    const int64_t t = t0 + row;
    const bool tv = t < a.T;
    int kept[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) kept[j] = (j < a.k) ? a.idx[(int64_t)rows[row] * a.k + j] : -1;
    const float th0 = a.thr[2 * (int64_t)rows[row]], th1 = a.thr[2 * (int64_t)rows[row] + 1];
    for (int cb = 0; cb < a.E; cb += 64) {
      const int nvalid = min(64, a.E - cb);
      const ChunkSpec cs{a.w_gate, a.w_noise, true, 0, cb, nvalid};
      __syncthreads();
      Proj<T>::run((const T*)a.x, a.d, rows, cs, P);
      __syncthreads();
      for (int j = sub; j < 64; j += 8) {
        float p = 0.f;
        if (j < nvalid && tv) {
          const int e = cb + j;
          float c = P[j >> 5][row][j & 31];
          if (a.bias) c += a.bias[e];
          float sp = softplus_f(P[2 + (j >> 5)][row][j & 31]);
          bool in = false;
#pragma unroll
          for (int q = 0; q < 8; ++q) in |= (kept[q] == e);
          float th = in ? th1 : th0;
          p = normal_cdf_f((c - th) / sp);
        }
        Q[row][j] = p;
      }
      __syncthreads();
      if (tid < 64 && tid < nvalid) {
        float s = acc[cb + tid];
        for (int r = 0; r < GATE_ROWS; ++r) s += Q[r][tid];
        acc[cb + tid] = s;
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < a.E; e += GATE_THREADS) a.part[(int64_t)blockIdx.x * a.E + e] = acc[e];
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
template <typename T>
static hipError_t launch_flat_t(const GateFlatArgs& a, hipStream_t s) {
  dim3 grid((unsigned)((a.T + GATE_ROWS - 1) / GATE_ROWS));
  if (a.k + 1 <= 3)
    hipLaunchKernelGGL((gate_flat_kernel<T, 3>), grid, dim3(GATE_THREADS), 0, s, a);
  else if (a.k + 1 <= 5)
    hipLaunchKernelGGL((gate_flat_kernel<T, 5>), grid, dim3(GATE_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((gate_flat_kernel<T, 9>), grid, dim3(GATE_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gate_flat(const GateFlatArgs& a, bool bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return bf16 ? launch_flat_t<bf16_t>(a, s) : launch_flat_t<float>(a, s);
}

template <typename T>
static hipError_t launch_group_t(const GateGroupArgs& a, int grid, hipStream_t s) {
  if (a.kpg + 1 <= 3)
    hipLaunchKernelGGL((gate_group_kernel<T, 3>), dim3(grid), dim3(GATE_THREADS), 0, s, a);
  else if (a.kpg + 1 <= 5)
    hipLaunchKernelGGL((gate_group_kernel<T, 5>), dim3(grid), dim3(GATE_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL((gate_group_kernel<T, 9>), dim3(grid), dim3(GATE_THREADS), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_gate_group(const GateGroupArgs& a, int grid, bool bf16, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  return bf16 ? launch_group_t<bf16_t>(a, grid, s) : launch_group_t<float>(a, grid, s);
}

int load_partial_blocks(int64_t T, int* tiles_per_block) {
  int64_t tiles = (T + GATE_ROWS - 1) / GATE_ROWS;
  int per = (int)std::max<int64_t>(1, (tiles + 511) / 512);  // at most ~512 partial rows
  *tiles_per_block = per;
  return (int)((tiles + per - 1) / per);
}

hipError_t launch_load_partial(const LoadArgs& a, int blocks, bool bf16, hipStream_t s) {
  if (blocks == 0) return hipSuccess;
  size_t sh = sizeof(float) * (size_t)a.E;
  if (bf16)
    hipLaunchKernelGGL((load_partial_kernel<bf16_t>), dim3(blocks), dim3(GATE_THREADS), sh, s, a);
  else
    hipLaunchKernelGGL((load_partial_kernel<float>), dim3(blocks), dim3(GATE_THREADS), sh, s, a);
  return hipGetLastError();
}

}  // namespace moe
