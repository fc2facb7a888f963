// Gate kernels: noisy scores, KeepTopK, softmax over the kept scores, and the
// smooth load estimate.
//
// Method ("MoE:稀疏门控混合专家", nengyongai.cn, sections 三 and 四):
//   clean_e = x . W_g[e] (+ bias_e)
//   H_e     = clean_e + eps_e * softplus(x . W_noise[e])   (noisy gate)
//   keep the k largest H_e (ties: lower e), softmax over the kept ones.
//
// A workgroup (8 waves) scores a tile of 32 rows (64 for large expert
// counts: RB = 2 blocks of 32, so that every table fragment fetched serves
// twice the rows) against the experts in blocks of 256: wave w computes the
// clean and the raw-noise scores of experts blk + 32w .. +31 for all the rows
// with v_mfma_f32_32x32x16_bf16 (one LDS input fragment feeds both tables'
// MFMAs; the table rows stream from global memory through a register ring).
// The scores stay in the MFMA accumulator layout: lane l holds expert
// (l mod 32) of its wave for the 16 rows acc_row(i, l) of each 32-row block.
// The noisy scores go through LDS to the selection step, where 16 (RB = 2:
// 8) lanes per row keep running top-(k+1) lists merged over DPP rows.  For
// the smooth load the clean scores and noise scales never leave the
// registers.  Outputs that feed the routing and the balance statistics (masks,
// partial sums) are written per 32-token block whatever the tile size.
#include <algorithm>

#include "gate_common.h"
#include "moe_kernels.h"

namespace moe {

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
  // Merge the lists of the TPR (16 or 8) lanes of a row, inside one DPP row:
  // every lane ends with the row's best K1 (value, expert) pairs in rank
  // order.  An expert sits in one lane's list only, so one lane pops per round.
  template <int TPR>
  __device__ __forceinline__ void merge(float* ov, int* oe) {
#pragma unroll
    for (int round = 0; round < K1; ++round) {
      float bv = v[0];
      int be = e[0];
      best_step<DPP_XOR1>(bv, be);
      best_step<DPP_XOR2>(bv, be);
      best_step<DPP_HALF_MIRROR>(bv, be);
      if constexpr (TPR == 16) best_step<DPP_MIRROR>(bv, be);
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

// Turn the merged top-(k+1) of a row (rank order) into the kept experts in
// ascending index order and their softmax gates; also the k-th and (k+1)-th
// scores.  Entries >= k are padding.
template <int K1>
__device__ __forceinline__ void kept_gates(const float* ov, const int* oe, int k, int E,
                                           int* ke, float* kg, float* kth, float* k1th) {
  float kv[K1];
#pragma unroll
  for (int j = 0; j < K1; ++j) {
    ke[j] = j < k ? oe[j] : 0x7fffffff;
    kv[j] = ov[j];
  }
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

// Per-row thresholds the load estimate needs, shared through LDS.
struct RowThr {
  float kth, k1th;
};

// One lane's load terms: sum over its 16 tile rows (register order) of
// Phi((clean - theta) / sp), then the two half-waves holding the same expert
// are added; rows at or past `valid` contribute 0.  Bit r of `kept` says
// whether tile row r keeps this lane's expert.  Identical in the gate and in
// the recompute kernel.
__device__ __forceinline__ float load_column_sum(const f32x16& clean, const f32x16& sp,
                                                 uint32_t kept, const RowThr* thr, int valid) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = acc_row(i, lane);
    const RowThr rt = thr[r];
    const float th = ((kept >> r) & 1u) ? rt.k1th : rt.kth;
    const float p = normal_cdf_f((clean[i] - th) * rcp_hw(sp[i]));
    s += r < valid ? p : 0.f;
  }
  return s + __shfl_xor(s, 32, 64);
}

// The scoring and selection of one tile of RB 32-row blocks against experts
// [0, E) of a table block (tb).  eps_at(i, e, out) gives the noise of expert
// e for the 16 accumulator rows of block i (all lanes call it together)
// (experts contiguous); Hs is the R x HLD score block in LDS.  On return every
// lane of a row's group holds the row's top-K1 in ov/oe, and cs/ss the clean
// scores (bias included) and noise scales of the last expert block.
template <typename T, int K1, bool NOISY, bool XLDS, int RB, typename EpsRow>
__device__ void score_tile(const TileX<T>& tx, int d, const GateTabs& tb,
                           const float* __restrict__ bias, int E, EpsRow eps_at, float* Hs,
                           float* ov, int* oe, f32x16 (&cs)[RB], f32x16 (&ss)[RB]) {
  using GT = GateTile<RB>;
  constexpr int TPR = GT::TPR, NQ = GT::NQ;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int row = tid / TPR, sub = tid % TPR;
  TopList<K1> L;
  L.init();
  for (int blk = 0; blk < E; blk += GATE_BLOCK_E) {
    const int e = blk + w * 32 + (lane & 31);
    const bool ev = e < E;
    // noise of this lane's (row, expert) pairs, requested before the MFMAs
    float ep[RB][16];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      if (NOISY) {
        eps_at(i, e, ep[i]);
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) ep[i][r] = 0.f;
      }
    }
    f32x16 ac[RB], ar[RB];
    BlockProj<T, NOISY, XLDS, RB>::run(tx, d, tb, blk, E, ac, ar);
    const float b = (bias && ev) ? bias[tb.row0 + e] : 0.f;
#pragma unroll
    for (int i = 0; i < RB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float c = ac[i][r] + b;
        float h = c;
        if (NOISY) {
          const float sp = softplus_f(ar[i][r]);
          h = noisy_score(c, ep[i][r], sp);
          ss[i][r] = sp;
        } else {
          ss[i][r] = 0.f;
        }
        cs[i][r] = c;
        Hs[(32 * i + acc_row(r, lane)) * HLD + w * 32 + (lane & 31)] = select_score(h);
      }
    __syncthreads();
    // lane `sub` of the row holds columns sub + TPR*q.  Only scores at or above
    // tau, the K1-th largest of the row's TPR lane maxima, can be among the
    // block's best K1 (K1 lanes hold a score >= tau); lanes whose maxima tie
    // leave together, which only lowers tau.
    const int nb = min(GATE_BLOCK_E, E - blk);
    float hv[NQ];
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int j = sub + TPR * q;
      hv[q] = j < nb ? Hs[row * HLD + j] : -INFINITY;
      mx = fmaxf(mx, hv[q]);
    }
    float tau = -INFINITY;
#pragma unroll
    for (int r = 0; r < K1; ++r) {
      tau = row_max<TPR>(mx);
      mx = mx == tau ? -INFINITY : mx;
    }
    uint32_t cand = 0u;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      if (sub + TPR * q < nb && hv[q] >= tau) cand |= 1u << q;
    while (cand) {
      const int q = __ffs(cand) - 1;
      cand &= cand - 1u;
      const int j = sub + TPR * q;
      L.insert(Hs[row * HLD + j], blk + j);
    }
    __syncthreads();
  }
  L.template merge<TPR>(ov, oe);
}

// ---------------------------------------------------------------------------
// Flat gate: tile = R = 32*RB consecutive tokens.  With a.part set (noisy
// gate, E <= GATE_FUSED_LOAD_MAX_E) the kernel also writes the smooth-load
// partial sums of each of its 32-token blocks; with a.imp_part (E <=
// GATE_FUSED_LOAD_MAX_E) their gate sums per expert (rows in ascending order);
// with a.bits their routing masks.  All use the masks sb[RB][E] in LDS (bit r
// of sb[i][e]: row 32i + r keeps expert e).
// Dynamic LDS: input tile (XLDS), score block Hs[R][HLD], masks.
// ---------------------------------------------------------------------------
template <typename T, int K1, bool NOISY, bool XLDS, int RB>
__global__ __launch_bounds__(GATE_THREADS) void gate_flat_kernel(GateFlatArgs a) {
  using GT = GateTile<RB>;
  constexpr int R = GT::R, TPR = GT::TPR;
  __shared__ int rows[R];
  __shared__ RowThr thr[R];
  __shared__ int kle[R][8];    // kept experts of each row
  __shared__ float klg[R][8];  // and their gates
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t t0 = (int64_t)blockIdx.x * R;
  const int64_t nblk = (a.T + GATE_ROWS - 1) / GATE_ROWS;  // 32-token blocks of the batch
  const int E = a.E;
  if (tid < R) rows[tid] = (int)min<int64_t>(t0 + tid, a.T - 1);
  const int xld = a.d + 8;
  const size_t xbytes = XLDS ? sizeof(bf16_t) * R * xld : 0;
  bf16_t* Xs = reinterpret_cast<bf16_t*>(dyn);
  float* Hs = reinterpret_cast<float*>(dyn + xbytes);
  uint32_t* sb = reinterpret_cast<uint32_t*>(dyn + xbytes + sizeof(float) * R * HLD);
  const bool masks = a.bits || (NOISY && a.part) || a.imp_part;
  if (masks)
    for (int i = tid; i < RB * E; i += GATE_THREADS) sb[i] = 0u;
  __syncthreads();
  if (XLDS) load_x_tile((const bf16_t*)a.x, a.d, rows, R, Xs, xld);
  __syncthreads();
  const TileX<T> tx{(const T*)a.x, rows, XLDS ? Xs : nullptr, xld};
  const NoiseSrc& noise = a.noise;
  auto eps_row = [&](int i, int e, float (&out)[16]) {
    noise.rows16(0, 1, e, E, [&](int r) { return rows[32 * i + acc_row(r, threadIdx.x & 63)]; }, out);
  };
  float ov[K1];
  int oe[K1];
  f32x16 cs[RB], ss[RB];
  const GateTabs tb{a.w_gate, a.w_noise, 0, (const bf16_t*)a.w_pack, 0, a.pack_nt};
  score_tile<T, K1, NOISY, XLDS, RB>(tx, a.d, tb, a.bias, E, eps_row, Hs, ov, oe, cs, ss);
  int ke[K1];
  float kg[K1], kth, k1th;
  kept_gates<K1>(ov, oe, a.k, E, ke, kg, &kth, &k1th);
  const int row = tid / TPR;
  const int64_t t = t0 + row;
  if (tid % TPR == 0) {
    if (t < a.T) {
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
      if (masks) {
#pragma unroll
        for (int j = 0; j < K1; ++j)
          if (j < a.k && (unsigned)ke[j] < (unsigned)E)
            atomicOr(&sb[(row >> 5) * E + ke[j]], 1u << (row & 31));
      }
    }
    thr[row].kth = kth;
    thr[row].k1th = k1th;
#pragma unroll
    for (int j = 0; j < K1; ++j) {
      if (j < a.k && j < 8) {
        kle[row][j] = ke[j];
        klg[row][j] = kg[j];
      }
    }
  }
  if (masks) __syncthreads();
#pragma unroll
  for (int hb = 0; hb < RB; ++hb) {
    const int64_t blk = (int64_t)blockIdx.x * RB + hb;  // 32-token block
    if (blk >= nblk) break;
    if (a.imp_part) {
      for (int e = tid; e < E; e += GATE_THREADS) {
        uint32_t m = sb[hb * E + e];
        float s = 0.f;
        while (m) {
          const int r = 32 * hb + __ffs(m) - 1;
          m &= m - 1u;
          for (int j = 0; j < a.k; ++j)
            if (kle[r][j] == e) s += klg[r][j];
        }
        a.imp_part[blk * E + e] = s;
      }
    }
    if (a.bits)
      for (int i = tid; i < E; i += GATE_THREADS) a.bits[blk * E + i] = sb[hb * E + i];
    if (NOISY && a.part) {
      const int e = (tid >> 6) * 32 + (lane & 31);
      const int valid = (int)max<int64_t>(0, min<int64_t>(GATE_ROWS, a.T - blk * GATE_ROWS));
      const uint32_t kept = e < E ? sb[hb * E + e] : 0u;
      const float s = load_column_sum(cs[hb], ss[hb], kept, thr + 32 * hb, valid);
      if (lane < 32 && e < E) a.part[blk * E + e] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Secondary gate of the hierarchy: rows are the (token, kept group) pairs of
// one group g, taken from the group routing (perm_g, offsets_g); tile i of
// group g covers positions offsets_g[g] + 32*(i - tiles_g[g]) onward.
// Writes the final experts g*Eg + j and gates gate_p * gate_s directly.
// Dynamic LDS: input tile (XLDS), score block Hs[32][HLD].
// ---------------------------------------------------------------------------
template <typename T, int K1, bool NOISY, bool XLDS, int RB>
__global__ __launch_bounds__(GATE_THREADS) void gate_group_kernel(GateGroupArgs a) {
  constexpr int TPR = GateTile<RB>::TPR, R = GateTile<RB>::R;
  __shared__ int rows[R];
  __shared__ int asg[R];
  __shared__ int s_g, s_p0, s_n;
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int tid = threadIdx.x;
  if (tid == 0) {
    int q = blockIdx.x, g = -1;
    for (int i = 0; i < a.G; ++i)
      if (q >= a.tiles_g[i] && q < a.tiles_g[i + 1]) g = i;
    s_g = g;
    if (g >= 0) {
      int p0 = a.offsets_g[g] + R * (q - a.tiles_g[g]);
      s_p0 = p0;
      s_n = min(R, a.offsets_g[g + 1] - p0);
    }
  }
  __syncthreads();
  const int g = s_g;
  if (g < 0) return;
  const int p0 = s_p0, n = s_n;
  if (tid < R) {
    int as = a.perm_g[p0 + min(tid, n - 1)];
    asg[tid] = as;
    rows[tid] = as / a.kg;
  }
  __syncthreads();
  const int xld = a.d + 8;
  const size_t xbytes = XLDS ? sizeof(bf16_t) * R * xld : 0;
  bf16_t* Xs = reinterpret_cast<bf16_t*>(dyn);
  float* Hs = reinterpret_cast<float*>(dyn + xbytes);
  if (XLDS) load_x_tile((const bf16_t*)a.x, a.d, rows, R, Xs, xld);
  __syncthreads();
  const TileX<T> tx{(const T*)a.x, rows, XLDS ? Xs : nullptr, xld};
  const int Eg = a.Eg, G = a.G;
  const NoiseSrc& noise = a.noise;
  auto eps_row = [&](int i, int j, float (&out)[16]) {
    noise.rows16(g, G, j, Eg, [&](int r) { return rows[32 * i + acc_row(r, threadIdx.x & 63)]; }, out);
  };
  float ov[K1];
  int oe[K1];
  f32x16 cs[RB], ss[RB];
  const GateTabs tb{a.w_gate, a.w_noise, g * Eg, (const bf16_t*)a.w_pack,
                    g * ((Eg + 31) / 32), a.pack_nt};
  score_tile<T, K1, NOISY, XLDS, RB>(tx, a.d, tb, nullptr, Eg, eps_row, Hs, ov, oe, cs, ss);
  const int row = tid / TPR;
  if (tid % TPR == 0 && row < n) {
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
// the gate's thresholds.  Workgroup b covers tokens [R b, R b + R), R = 32*RB,
// and writes for each of its 32-token blocks c
//   part[c][e] = sum over the block's rows of
//                Phi((clean[t,e] - theta[t,e]) / softplus(raw[t,e]))
// with theta = thr[t][1] if e is kept by t, else thr[t][0]: the same terms,
// in the same order, as the gate kernel's fused variant.
// Dynamic LDS: input tile (XLDS), masks sb[RB][E].
// ---------------------------------------------------------------------------
template <typename T, bool XLDS, int RB>
__global__ __launch_bounds__(GATE_THREADS) void load_partial_kernel(LoadArgs a) {
  constexpr int R = GateTile<RB>::R;
  __shared__ int rows[R];
  __shared__ RowThr thr[R];
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * R;
  const int64_t nblk = (a.T + GATE_ROWS - 1) / GATE_ROWS;
  const int xld = a.d + 8;
  bf16_t* Xs = reinterpret_cast<bf16_t*>(dyn);
  uint32_t* sb = reinterpret_cast<uint32_t*>(dyn + (XLDS ? sizeof(bf16_t) * R * xld : 0));
  for (int i = tid; i < RB * a.E; i += GATE_THREADS) sb[i] = 0u;
  if (tid < R) {
    const int r = (int)min<int64_t>(t0 + tid, a.T - 1);
    rows[tid] = r;
    thr[tid].kth = a.thr[2 * (int64_t)r];
    thr[tid].k1th = a.thr[2 * (int64_t)r + 1];
  }
  __syncthreads();
  // kept-expert masks of the tile's valid rows
  for (int i = tid; i < R * a.k; i += GATE_THREADS) {
    const int r = i / a.k;
    const int e = t0 + r < a.T ? a.idx[(t0 + r) * a.k + i % a.k] : -1;
    if ((unsigned)e < (unsigned)a.E) atomicOr(&sb[(r >> 5) * a.E + e], 1u << (r & 31));
  }
  if (XLDS) load_x_tile((const bf16_t*)a.x, a.d, rows, R, Xs, xld);
  __syncthreads();
  const TileX<T> tx{(const T*)a.x, rows, XLDS ? Xs : nullptr, xld};
  const GateTabs tb{a.w_gate, a.w_noise, 0, (const bf16_t*)a.w_pack, 0, 2};
  for (int blk = 0; blk < a.E; blk += GATE_BLOCK_E) {
    const int e = blk + w * 32 + (lane & 31);
    f32x16 ac[RB], ar[RB];
    BlockProj<T, true, XLDS, RB>::run(tx, a.d, tb, blk, a.E, ac, ar);
    const float b = (a.bias && e < a.E) ? a.bias[e] : 0.f;
#pragma unroll
    for (int hb = 0; hb < RB; ++hb) {
      const int64_t cb = (int64_t)blockIdx.x * RB + hb;  // 32-token block
      f32x16 cs, ss;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        cs[i] = ac[hb][i] + b;
        ss[i] = softplus_f(ar[hb][i]);
      }
      const int valid = (int)max<int64_t>(0, min<int64_t>(GATE_ROWS, a.T - cb * GATE_ROWS));
      const uint32_t kept = e < a.E ? sb[hb * a.E + e] : 0u;
      const float s = load_column_sum(cs, ss, kept, thr + 32 * hb, valid);
      if (lane < 32 && e < a.E && cb < nblk) a.part[cb * a.E + e] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------
static bool xtile_in_lds(bool bf16, int d) { return bf16 && d <= GATE_XLDS_MAX_D; }

static size_t xtile_bytes(bool bf16, int d, int rows) {
  return xtile_in_lds(bf16, d) ? sizeof(bf16_t) * rows * (size_t)(d + 8) : 0;
}

// Dynamic LDS the kernels may take (the static arrays come on top).
constexpr size_t GATE_DYN_LDS_MAX = 150 * 1024;

// Raise a kernel's dynamic LDS limit when needed; `done` caches the largest
// size already granted to that kernel.
template <typename K>
static hipError_t set_lds(K kernel, size_t bytes, size_t* done) {
  if (bytes <= 32768 || bytes <= *done) return hipSuccess;
  hipError_t err = hipFuncSetAttribute((const void*)kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err == hipSuccess) *done = bytes;
  return err;
}

// Tiles of 64 rows for large expert counts (each table fragment serves twice
// the rows), when the input tile is in LDS and everything fits.
static size_t flat_lds(bool bf16, int d, int E, bool masks, int rb) {
  return xtile_bytes(bf16, d, 32 * rb) + sizeof(float) * 32 * rb * HLD +
         (masks ? sizeof(uint32_t) * (size_t)rb * E : 0);
}
static int flat_rb(bool bf16, int d, int E, bool masks) {
  return (xtile_in_lds(bf16, d) && E >= 2 * GATE_BLOCK_E &&
          flat_lds(bf16, d, E, masks, 2) <= GATE_DYN_LDS_MAX) ? 2 : 1;
}
static size_t load_lds(bool bf16, int d, int E, int rb) {
  return xtile_bytes(bf16, d, 32 * rb) + sizeof(uint32_t) * (size_t)rb * E;
}
static int load_rb(bool bf16, int d, int E) {
  return (xtile_in_lds(bf16, d) && E >= 2 * GATE_BLOCK_E &&
          load_lds(bf16, d, E, 2) <= GATE_DYN_LDS_MAX) ? 2 : 1;
}

template <typename T, int K1, bool NOISY, bool XLDS, int RB>
static hipError_t launch_flat_v(const GateFlatArgs& a, size_t sh, hipStream_t s) {
  static size_t granted = 0;
  hipError_t err = set_lds(gate_flat_kernel<T, K1, NOISY, XLDS, RB>, sh, &granted);
  if (err != hipSuccess) return err;
  constexpr int R = GateTile<RB>::R;
  dim3 grid((unsigned)((a.T + R - 1) / R));
  hipLaunchKernelGGL((gate_flat_kernel<T, K1, NOISY, XLDS, RB>), grid, dim3(GATE_THREADS), sh, s,
                     a);
  return hipGetLastError();
}

template <typename T, int K1, bool NOISY>
static hipError_t launch_flat_n(const GateFlatArgs& a, bool masks, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (xtile_in_lds(true, a.d)) {
      if (flat_rb(true, a.d, a.E, masks) == 2)
        return launch_flat_v<T, K1, NOISY, true, 2>(a, flat_lds(true, a.d, a.E, masks, 2), s);
      return launch_flat_v<T, K1, NOISY, true, 1>(a, flat_lds(true, a.d, a.E, masks, 1), s);
    }
  }
  return launch_flat_v<T, K1, NOISY, false, 1>(a, flat_lds(sizeof(T) == 2, a.d, a.E, masks, 1), s);
}

template <typename T, int K1>
static hipError_t launch_flat_k(const GateFlatArgs& a, bool noisy, hipStream_t s) {
  const bool masks = a.bits || (noisy && a.part) || a.imp_part;
  return noisy ? launch_flat_n<T, K1, true>(a, masks, s) : launch_flat_n<T, K1, false>(a, masks, s);
}

template <typename T>
static hipError_t launch_flat_t(const GateFlatArgs& a, hipStream_t s) {
  const bool noisy = a.noise.on() && a.w_noise != nullptr;
  if (a.k + 1 <= 3) return launch_flat_k<T, 3>(a, noisy, s);
  if (a.k + 1 <= 5) return launch_flat_k<T, 5>(a, noisy, s);
  return launch_flat_k<T, 9>(a, noisy, s);
}

bool gate_fuses_load(int E) { return E <= GATE_FUSED_LOAD_MAX_E; }

hipError_t launch_gate_flat(const GateFlatArgs& a, bool bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  return bf16 ? launch_flat_t<bf16_t>(a, s) : launch_flat_t<float>(a, s);
}

template <typename T, int K1, bool NOISY, bool XLDS, int RB>
static hipError_t launch_group_r(const GateGroupArgs& a, int grid, hipStream_t s) {
  const size_t sh = xtile_bytes(sizeof(T) == 2, a.d, 32 * RB) + sizeof(float) * 32 * RB * HLD;
  static size_t granted = 0;
  hipError_t err = set_lds(gate_group_kernel<T, K1, NOISY, XLDS, RB>, sh, &granted);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((gate_group_kernel<T, K1, NOISY, XLDS, RB>), dim3(grid), dim3(GATE_THREADS),
                     sh, s, a);
  return hipGetLastError();
}

// 64-row tiles (RB = 2) when the launch asks for them (bf16 with the input
// tile in LDS, see gate_group_tile_rows): every table fragment fetched then
// serves twice the rows
template <typename T, int K1, bool NOISY, bool XLDS>
static hipError_t launch_group_v(const GateGroupArgs& a, int grid, size_t, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && XLDS) {
    if (a.tile_rows == 64) return launch_group_r<T, K1, NOISY, XLDS, 2>(a, grid, s);
  } else {
    if (a.tile_rows != 32) return hipErrorInvalidValue;
  }
  return launch_group_r<T, K1, NOISY, XLDS, 1>(a, grid, s);
}

template <typename T, int K1>
static hipError_t launch_group_k(const GateGroupArgs& a, int grid, size_t sh, hipStream_t s) {
  const bool noisy = a.noise.on() && a.w_noise != nullptr;
  if constexpr (sizeof(T) == 2) {
    if (xtile_in_lds(true, a.d))
      return noisy ? launch_group_v<T, K1, true, true>(a, grid, sh, s)
                   : launch_group_v<T, K1, false, true>(a, grid, sh, s);
  }
  return noisy ? launch_group_v<T, K1, true, false>(a, grid, sh, s)
               : launch_group_v<T, K1, false, false>(a, grid, sh, s);
}

template <typename T>
static hipError_t launch_group_t(const GateGroupArgs& a, int grid, hipStream_t s) {
  const size_t sh = xtile_bytes(sizeof(T) == 2, a.d, GATE_ROWS) + sizeof(float) * GATE_ROWS * HLD;
  if (a.kpg + 1 <= 3) return launch_group_k<T, 3>(a, grid, sh, s);
  if (a.kpg + 1 <= 5) return launch_group_k<T, 5>(a, grid, sh, s);
  return launch_group_k<T, 9>(a, grid, sh, s);
}

int gate_group_tile_rows(bool bf16, int d, int64_t rows, int G) {
  return bf16 && xtile_in_lds(true, d) && rows >= 64 * (int64_t)G ? 64 : 32;
}

hipError_t launch_gate_group(const GateGroupArgs& a, int grid, bool bf16, hipStream_t s) {
  if (grid == 0) return hipSuccess;
  if (a.tile_rows != 32 && a.tile_rows != 64) return hipErrorInvalidValue;
  return bf16 ? launch_group_t<bf16_t>(a, grid, s) : launch_group_t<float>(a, grid, s);
}

// packed[((((g*BG + b)*NG + G)*nt + t)*4 + j)*64 + l] (16 bytes each) =
//   table t, row g*eg + min(32b + l%32, eg-1), columns 64G + 32(l/32) + 8j ..+7
// with BG = ceil(eg/32), NG = d/64: the fragment lane l of the wave scoring
// block b loads at step j of column group G.
__global__ __launch_bounds__(256) void pack_gate_kernel(const bf16_t* wg, const bf16_t* wn,
                                                        int ng, int eg, int d, int nt,
                                                        bf16_t* out) {
  const int BG = (eg + 31) / 32, NG = d / 64;
  const int64_t n = (int64_t)ng * BG * NG * nt * 4 * 64;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  int64_t r = i;
  const int l = (int)(r % 64); r /= 64;
  const int j = (int)(r % 4); r /= 4;
  const int t = (int)(r % nt); r /= nt;
  const int G = (int)(r % NG); r /= NG;
  const int b = (int)(r % BG);
  const int g = (int)(r / BG);
  const int64_t row = (int64_t)g * eg + min(32 * b + (l & 31), eg - 1);
  const int col = 64 * G + 32 * (l >> 5) + 8 * j;
  const bf16_t* src = (t == 0 ? wg : wn) + row * d + col;
  *reinterpret_cast<u32x4*>(out + i * 8) = *reinterpret_cast<const u32x4*>(src);
}

bool gate_pack_supported(bool bf16, int d) { return bf16 && d > 0 && d % 64 == 0; }

size_t gate_packed_bytes(int ng, int eg, int d, int nt) {
  return sizeof(bf16_t) * (size_t)ng * (size_t)((eg + 31) / 32) * 32 * (size_t)d * nt;
}

hipError_t launch_pack_gate(const void* w_gate, const void* w_noise, int ng, int eg, int d, int nt,
                            void* out, hipStream_t s) {
  const int64_t n = (int64_t)ng * ((eg + 31) / 32) * (d / 64) * nt * 4 * 64;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_gate_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const bf16_t*)w_gate, (const bf16_t*)w_noise, ng, eg, d, nt, (bf16_t*)out);
  return hipGetLastError();
}

int load_partial_blocks(int64_t T) { return (int)((T + GATE_ROWS - 1) / GATE_ROWS); }

template <typename T, bool XLDS, int RB>
static hipError_t launch_load_v(const LoadArgs& a, size_t sh, hipStream_t s) {
  static size_t granted = 0;
  hipError_t err = set_lds(load_partial_kernel<T, XLDS, RB>, sh, &granted);
  if (err != hipSuccess) return err;
  constexpr int R = GateTile<RB>::R;
  hipLaunchKernelGGL((load_partial_kernel<T, XLDS, RB>), dim3((unsigned)((a.T + R - 1) / R)),
                     dim3(GATE_THREADS), sh, s, a);
  return hipGetLastError();
}

hipError_t launch_load_partial(const LoadArgs& a, bool bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (!bf16) return launch_load_v<float, false, 1>(a, load_lds(false, a.d, a.E, 1), s);
  if (!xtile_in_lds(true, a.d))
    return launch_load_v<bf16_t, false, 1>(a, load_lds(true, a.d, a.E, 1), s);
  if (load_rb(true, a.d, a.E) == 2)
    return launch_load_v<bf16_t, true, 2>(a, load_lds(true, a.d, a.E, 2), s);
  return launch_load_v<bf16_t, true, 1>(a, load_lds(true, a.d, a.E, 1), s);
}

}  // namespace moe
