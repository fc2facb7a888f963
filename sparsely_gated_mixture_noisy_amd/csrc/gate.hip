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

// bf16 projection with the 32-row input tile in LDS (row stride xld): the
// A operand comes from LDS, the table rows stream from global memory through
// a 16-deep register ring so that many loads are in flight per wave.
__device__ __forceinline__ void proj_lds(const bf16_t* Xs, int xld, int d, const ChunkSpec& cs,
                                         ProjTile* P) {
  constexpr int RING = 16;
  const int lane = threadIdx.x & 63, b = threadIdx.x >> 6;
  const int c = lane & 31, kh = (lane >> 5) * 8;
  const BlockCols bc = block_cols(b, cs.wg, cs.wn, cs.noisy, cs.tab_row0, cs.cb, cs.nvalid);
  const int trow = c < bc.valid ? bc.row0 + c : bc.safe;
  const bf16_t* wp = (const bf16_t*)bc.tab + (int64_t)trow * d + kh;
  const bf16_t* xp = Xs + c * xld + kh;
  const int KS = d / 16;
  u32x4 rb[RING];
#pragma unroll
  for (int i = 0; i < RING; ++i)
    rb[i] = i < KS ? *reinterpret_cast<const u32x4*>(wp + i * 16) : u32x4{0u, 0u, 0u, 0u};
  f32x16 acc = {};
  for (int g = 0; g < KS; g += RING) {
#pragma unroll
    for (int i = 0; i < RING; ++i) {
      const int ks = g + i;
      if (ks < KS) {
        const bf16x8 bv = __builtin_bit_cast(bf16x8, rb[i]);
        if (ks + RING < KS) rb[i] = *reinterpret_cast<const u32x4*>(wp + (ks + RING) * 16);
        const bf16x8 av = *reinterpret_cast<const bf16x8*>(xp + ks * 16);
        acc = mfma32(av, bv, acc);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    P[b][r][c] = acc[i];
  }
}

// Where a tile's input rows come from: global memory (rows[] tokens) or, for
// bf16 with d <= 1024, an LDS copy Xs of the 32 rows.
template <typename T>
struct TileX {
  const T* x;
  const int* rows;
  const bf16_t* Xs;  // null: read x directly
  int xld;
};

template <typename T>
__device__ __forceinline__ void project(const TileX<T>& tx, int d, const ChunkSpec& cs,
                                        ProjTile* P) {
  if constexpr (sizeof(T) == 2) {
    if (tx.Xs) {
      proj_lds(tx.Xs, tx.xld, d, cs, P);
      return;
    }
  }
  Proj<T>::run(tx.x, d, tx.rows, cs, P);
}

// Copy the 32 input rows of a tile to LDS (bf16 only, d % 8 == 0).
__device__ __forceinline__ void load_x_tile(const bf16_t* x, int d, const int* rows, bf16_t* Xs,
                                            int xld) {
  const int cpr = d / 8;
  for (int c = threadIdx.x; c < GATE_ROWS * cpr; c += GATE_THREADS) {
    const int r = c / cpr, cc = (c % cpr) * 8;
    *reinterpret_cast<u32x4*>(Xs + r * xld + cc) =
        *reinterpret_cast<const u32x4*>(x + (int64_t)rows[r] * d + cc);
  }
}

constexpr int GATE_XLDS_MAX_D = 1024;  // input tile in LDS up to this d_model

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
// pointer (unused when !noisy).  With keep != null the clean score and the
// noise scale of every (row, expert) are also kept: keep[r*E+e] and
// keep[32*E + r*E+e].
template <typename T, int K1>
__device__ void score_tile(const TileX<T>& tx, int d, const void* wg, const void* wn,
                           const float* __restrict__ bias, int tab_row0, int E, const float* erow,
                           bool noisy, ProjTile* P, TopList<K1>& L, float* keep) {
  const int tid = threadIdx.x;
  const int row = tid >> 3, sub = tid & 7;
  const int ce = noisy ? 64 : 128;  // experts per chunk
  for (int cb = 0; cb < E; cb += ce) {
    const int nvalid = min(ce, E - cb);
    const ChunkSpec cs{wg, wn, noisy, tab_row0, cb, nvalid};
    __syncthreads();  // P is free
    project<T>(tx, d, cs, P);
    __syncthreads();
    for (int j = sub; j < nvalid; j += 8) {
      const int e = cb + j;
      float c = P[j >> 5][row][j & 31];
      if (bias) c += bias[tab_row0 + e];
      float h = c;
      if (noisy) {
        const float sp = softplus_f(P[2 + (j >> 5)][row][j & 31]);
        h = c + erow[e] * sp;
        if (keep) {
          keep[row * E + e] = c;
          keep[GATE_ROWS * E + row * E + e] = sp;
        }
      }
      L.insert(h, e);
    }
  }
}

// One row's load term of expert e: Phi((clean - theta) / sp), theta the k-th
// largest noisy score among the other experts.
__device__ __forceinline__ float load_term(float clean, float sp, bool kept, float kth,
                                           float k1th) {
  const float th = kept ? k1th : kth;
  return normal_cdf_f((clean - th) / sp);
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
// Flat gate: tile = 32 consecutive tokens.  With a.part set (noisy gate,
// E <= 256) the kernel also produces the tile's row of smooth-load partial
// sums, from the clean scores and noise scales it kept in LDS.
// ---------------------------------------------------------------------------
template <typename T, int K1>
__global__ __launch_bounds__(GATE_THREADS) void gate_flat_kernel(GateFlatArgs a) {
  __shared__ ProjTile P[4];
  __shared__ int rows[GATE_ROWS];
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * GATE_ROWS;
  if (tid < GATE_ROWS) rows[tid] = (int)min<int64_t>(t0 + tid, a.T - 1);
  __syncthreads();
  const bool xl = sizeof(T) == 2 && a.d <= GATE_XLDS_MAX_D;
  const int xld = a.d + 8;
  bf16_t* Xs = xl ? reinterpret_cast<bf16_t*>(dyn) : nullptr;
  float* keep = a.part ? reinterpret_cast<float*>(dyn + (xl ? sizeof(bf16_t) * GATE_ROWS * xld : 0))
                       : nullptr;
  if (xl) load_x_tile((const bf16_t*)a.x, a.d, rows, Xs, xld);
  const TileX<T> tx{(const T*)a.x, rows, Xs, xld};
  const int row = tid >> 3;
  const int64_t t = t0 + row;
  const bool noisy = a.eps != nullptr && a.w_noise != nullptr;
  const float* erow = noisy ? a.eps + (int64_t)rows[row] * a.E : nullptr;
  TopList<K1> L;
  L.init();
  score_tile<T, K1>(tx, a.d, a.w_gate, a.w_noise, a.bias, 0, a.E, erow, noisy, P, L, keep);
  float ov[K1];
  int oe[K1];
  L.merge8(ov, oe);
  int ke[K1];
  float kg[K1], kth, k1th;
  kept_gates<K1>(ov, oe, a.k, a.E, ke, kg, &kth, &k1th);
  if ((tid & 7) == 0 && t < a.T) {
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
  if (keep) {
    // this row's load terms, in place of the clean scores (0 past the batch)
    for (int e = tid & 7; e < a.E; e += 8) {
      bool in = false;
#pragma unroll
      for (int j = 0; j < K1; ++j) in |= (j < a.k && ke[j] == e);
      const float v = load_term(keep[row * a.E + e], keep[GATE_ROWS * a.E + row * a.E + e], in,
                                kth, k1th);
      keep[row * a.E + e] = t < a.T ? v : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < a.E; e += GATE_THREADS) {
      float sum = 0.f;
      for (int r = 0; r < GATE_ROWS; ++r) sum += keep[r * a.E + e];
      a.part[(int64_t)blockIdx.x * a.E + e] = sum;
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
  extern __shared__ __attribute__((aligned(16))) char dyn[];
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
  const bool xl = sizeof(T) == 2 && a.d <= GATE_XLDS_MAX_D;
  const int xld = a.d + 8;
  bf16_t* Xs = xl ? reinterpret_cast<bf16_t*>(dyn) : nullptr;
  if (xl) load_x_tile((const bf16_t*)a.x, a.d, rows, Xs, xld);
  const TileX<T> tx{(const T*)a.x, rows, Xs, xld};
  const int row = tid >> 3;
  const int Eg = a.Eg;
  const bool noisy = a.eps != nullptr && a.w_noise != nullptr;
  const float* erow = noisy ? a.eps + ((int64_t)rows[row] * a.G + g) * Eg : nullptr;
  TopList<K1> L;
  L.init();
  score_tile<T, K1>(tx, a.d, a.w_gate, a.w_noise, nullptr, g * Eg, Eg, erow, noisy, P, L,
                    nullptr);
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
// Smooth load estimate (flat noisy gate), recomputing the projections from
// the gate's thresholds.  Workgroup b covers tokens [32b, 32b+32) and writes
//   part[b][e] = sum over its rows (ascending) of
//                Phi((clean[t,e] - theta[t,e]) / softplus(raw[t,e]))
// with theta = thr[t][1] if e is kept by t, else thr[t][0]: the same terms,
// in the same order, as the gate kernel's fused variant.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(GATE_THREADS) void load_partial_kernel(LoadArgs a) {
  __shared__ ProjTile P[4];
  __shared__ int rows[GATE_ROWS];
  __shared__ float Q[GATE_ROWS][65];
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int tid = threadIdx.x;
  const int row = tid >> 3, sub = tid & 7;
  const int64_t t0 = (int64_t)blockIdx.x * GATE_ROWS;
  if (tid < GATE_ROWS) rows[tid] = (int)min<int64_t>(t0 + tid, a.T - 1);
  __syncthreads();
  const bool xl = sizeof(T) == 2 && a.d <= GATE_XLDS_MAX_D;
  const int xld = a.d + 8;
  bf16_t* Xs = xl ? reinterpret_cast<bf16_t*>(dyn) : nullptr;
  if (xl) load_x_tile((const bf16_t*)a.x, a.d, rows, Xs, xld);
  const TileX<T> tx{(const T*)a.x, rows, Xs, xld};
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
    project<T>(tx, a.d, cs, P);
    __syncthreads();
    for (int j = sub; j < 64; j += 8) {
      float p = 0.f;
      if (j < nvalid && tv) {
        const int e = cb + j;
        float c = P[j >> 5][row][j & 31];
        if (a.bias) c += a.bias[e];
        const float sp = softplus_f(P[2 + (j >> 5)][row][j & 31]);
        bool in = false;
#pragma unroll
        for (int q = 0; q < 8; ++q) in |= (kept[q] == e);
        p = load_term(c, sp, in, th0, th1);
      }
      Q[row][j] = p;
    }
    __syncthreads();
    if (tid < nvalid) {
      float sum = 0.f;
      for (int r = 0; r < GATE_ROWS; ++r) sum += Q[r][tid];
      a.part[(int64_t)blockIdx.x * a.E + cb + tid] = sum;
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static size_t xtile_bytes(bool bf16, int d) {
  return (bf16 && d <= GATE_XLDS_MAX_D) ? sizeof(bf16_t) * GATE_ROWS * (size_t)(d + 8) : 0;
}

// Raise a kernel's dynamic LDS limit when needed; `done` caches the largest
// size already granted to that kernel.
template <typename K>
static hipError_t set_lds(K kernel, size_t bytes, size_t* done) {
  if (bytes <= 65536 || bytes <= *done) return hipSuccess;
  hipError_t err = hipFuncSetAttribute((const void*)kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err == hipSuccess) *done = bytes;
  return err;
}

template <typename T, int K1>
static hipError_t launch_flat_k(const GateFlatArgs& a, size_t sh, hipStream_t s) {
  static size_t granted = 0;
  hipError_t err = set_lds(gate_flat_kernel<T, K1>, sh, &granted);
  if (err != hipSuccess) return err;
  dim3 grid((unsigned)((a.T + GATE_ROWS - 1) / GATE_ROWS));
  hipLaunchKernelGGL((gate_flat_kernel<T, K1>), grid, dim3(GATE_THREADS), sh, s, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_flat_t(const GateFlatArgs& a, hipStream_t s) {
  size_t sh = xtile_bytes(sizeof(T) == 2, a.d);
  if (a.part) sh += sizeof(float) * 2 * GATE_ROWS * (size_t)a.E;
  if (a.k + 1 <= 3) return launch_flat_k<T, 3>(a, sh, s);
  if (a.k + 1 <= 5) return launch_flat_k<T, 5>(a, sh, s);
  return launch_flat_k<T, 9>(a, sh, s);
}

bool gate_fuses_load(int E) { return E <= GATE_FUSED_LOAD_MAX_E; }

hipError_t launch_gate_flat(const GateFlatArgs& a, bool bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return bf16 ? launch_flat_t<bf16_t>(a, s) : launch_flat_t<float>(a, s);
}

template <typename T, int K1>
static hipError_t launch_group_k(const GateGroupArgs& a, int grid, size_t sh, hipStream_t s) {
  static size_t granted = 0;
  hipError_t err = set_lds(gate_group_kernel<T, K1>, sh, &granted);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((gate_group_kernel<T, K1>), dim3(grid), dim3(GATE_THREADS), sh, s, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_group_t(const GateGroupArgs& a, int grid, hipStream_t s) {
  const size_t sh = xtile_bytes(sizeof(T) == 2, a.d);
  if (a.kpg + 1 <= 3) return launch_group_k<T, 3>(a, grid, sh, s);
  if (a.kpg + 1 <= 5) return launch_group_k<T, 5>(a, grid, sh, s);
  return launch_group_k<T, 9>(a, grid, sh, s);
}

hipError_t launch_gate_group(const GateGroupArgs& a, int grid, bool bf16, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  return bf16 ? launch_group_t<bf16_t>(a, grid, s) : launch_group_t<float>(a, grid, s);
}

int load_partial_blocks(int64_t T) { return (int)((T + GATE_ROWS - 1) / GATE_ROWS); }

hipError_t launch_load_partial(const LoadArgs& a, bool bf16, hipStream_t s) {
  const int blocks = load_partial_blocks(a.T);
  if (blocks == 0) return hipSuccess;
  const size_t sh = xtile_bytes(bf16, a.d);
  if (bf16) {
    static size_t granted = 0;
    hipError_t err = set_lds(load_partial_kernel<bf16_t>, sh, &granted);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((load_partial_kernel<bf16_t>), dim3(blocks), dim3(GATE_THREADS), sh, s, a);
  } else {
    hipLaunchKernelGGL((load_partial_kernel<float>), dim3(blocks), dim3(GATE_THREADS), sh, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
