// Expert FFNs over the routed rows.
//
// Expert e is a one-hidden-layer FFN ("MoE:稀疏门控混合专家", nengyongai.cn,
// section 二: 512 -> 1024 -> 512, ReLU); the SwiGLU variant of the Mixtral
// page ("MoE 混合专家：参数大、计算省", section 核心概念) uses gate/up/down
// tables.  Only the rows routed to an expert are evaluated: the grid walks a
// tile map built from the routing offsets, so experts with no rows cost
// nothing.
//
// bf16 path: two grouped GEMMs on MFMA (v_mfma_f32_32x32x16_bf16), both
// operands K-contiguous ([rows][K] activations, [N][K] weight tables):
//   hid[p]      = act(x[row p] W1_e^T (, x[row p] W3_e^T))   bf16, [A][h]
//   y_sorted[p] = hid[p] W2_e^T                              bf16, [A][d]
// 128x128 output tiles, K staged through LDS in 32-wide double-buffered
// slices, fp32 accumulation.
// fp32 path: one thread per output, fp32 FMA (small layers).
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int GM_BM = 128, GM_BN = 128, GM_BK = 32, GM_LD = GM_BK + 8;

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// EPI_RELU_BWD, EPI_SWIGLU_BWD: the backward's hidden layer (large tiles
// only); C2 holds dHid = dY W2_e on entry and gets dP (ReLU) or dA (SwiGLU),
// C3 gets dB, C gets the recomputed hidden activations
enum { EPI_NONE = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_RELU_BWD = 3, EPI_SWIGLU_BWD = 4 };

struct GemmArgs {
  const bf16_t* A;
  int64_t lda;
  const int32_t* perm;  // null: source row of position p is p; else perm[p] / k
  int k;
  const bf16_t* B;      // [E][N][K]
  const bf16_t* B3;     // [E][N][K] (SwiGLU up) or null
  int N, K;
  const int32_t* offsets;  // [E+1]
  const int32_t* tiles;    // [E+1] tiles of GM_BM rows
  int E;
  bf16_t* C;               // [A][ldc]
  int64_t ldc;
  int ncol;                // ceil(N / GM_BN)
  bf16_t* C2 = nullptr;    // backward epilogues: [A][ldc], dHid in, dP / dA out
  bf16_t* C3 = nullptr;    // SwiGLU backward: dB [A][ldc]
  // large tiles only: a second operand pair (same layouts) whose product is
  // added, K running over A, B first and then A2, B2
  const bf16_t* A2 = nullptr;
  const bf16_t* B2 = nullptr;
  // per-expert table gradients (large tiles, WGT): C_e [M][N] = sum over
  // the positions p of expert e of A[p][m] B[p][n]; positions past an
  // expert's rows read the zero row (at least max(M, N) zeros)
  // The tile enumeration runs over wrows row tiles per expert against ncol
  // column tiles; with wswap its rows are the output's column tiles and its
  // columns the output's row tiles
  int M = 0, wrows = 0, wswap = 0;
  const bf16_t* zero = nullptr;
};

// Expert owning tile q: the largest e with tiles[e] <= q (tiles non-decreasing).
__device__ __forceinline__ int expert_of_tile(const int32_t* tiles, int E, int q) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (tiles[mid] <= q) lo = mid; else hi = mid - 1;
  }
  return lo;
}

template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemmArgs g) {
  constexpr bool SW = (EPI == EPI_SWIGLU);
  __shared__ __attribute__((aligned(16))) bf16_t As[2][GM_BM][GM_LD];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][GM_BN][GM_LD];
  constexpr int B3B = SW ? 2 : 1, B3R = SW ? GM_BN : 1;
  __shared__ __attribute__((aligned(16))) bf16_t B3s[B3B][B3R][GM_LD];
  __shared__ int s_e, s_row0, s_m;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = blockIdx.x / g.ncol, ct = blockIdx.x % g.ncol;
  if (tid == 0) {
    int Q = g.tiles[g.E];
    if (q < Q) {
      int e = expert_of_tile(g.tiles, g.E, q);
      int row0 = g.offsets[e] + (q - g.tiles[e]) * GM_BM;
      s_e = e;
      s_row0 = row0;
      s_m = min(GM_BM, g.offsets[e + 1] - row0);
    } else {
      s_e = -1;
    }
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int row0 = s_row0, m = s_m;
  const int n0 = ct * GM_BN;

  // global -> LDS assignment: 2 chunks of 16 bytes per thread per operand
  const int lrow = tid >> 2, lk = (tid & 3) * 8;
  const bf16_t* ap[2];
  const bf16_t* bp[2];
  const bf16_t* b3p[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    int r = lrow + 64 * i;
    int p = row0 + min(r, m - 1);
    int64_t src = g.perm ? (int64_t)(g.perm[p] / g.k) : (int64_t)p;
    ap[i] = g.A + src * g.lda + lk;
    int n = min(n0 + r, g.N - 1);
    bp[i] = g.B + ((int64_t)e * g.N + n) * g.K + lk;
    b3p[i] = SW ? g.B3 + ((int64_t)e * g.N + n) * g.K + lk : g.B;
  }

  const int wm = w >> 1, wn = w & 1;
  const bool active = wm * 64 < m;
  f32x16 acc[2][2], acc3[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = f32x16{};
      acc3[i][j] = f32x16{};
    }

  u32x4 ra[2], rb[2], rb3[2];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i] = *reinterpret_cast<const u32x4*>(ap[i] + k0);
      rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + k0);
      if constexpr (SW) rb3[i] = *reinterpret_cast<const u32x4*>(b3p[i] + k0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<u32x4*>(&As[buf][lrow + 64 * i][lk]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][lrow + 64 * i][lk]) = rb[i];
      if constexpr (SW) *reinterpret_cast<u32x4*>(&B3s[buf][lrow + 64 * i][lk]) = rb3[i];
    }
  };

  const int nk = g.K / GM_BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int fr = lane & 31, fk = (lane >> 5) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * GM_BK);
    if (active) {
#pragma unroll
      for (int ks = 0; ks < GM_BK; ks += 16) {
        bf16x8 af[2], bf[2], b3f[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          af[i] = *reinterpret_cast<const bf16x8*>(&As[buf][wm * 64 + i * 32 + fr][ks + fk]);
          bf[i] = *reinterpret_cast<const bf16x8*>(&Bs[buf][wn * 64 + i * 32 + fr][ks + fk]);
          if constexpr (SW)
            b3f[i] = *reinterpret_cast<const bf16x8*>(&B3s[buf][wn * 64 + i * 32 + fr][ks + fk]);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
            if constexpr (SW) acc3[i][j] = mfma32(af[i], b3f[j], acc3[i][j]);
          }
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  if (!active) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = n0 + wn * 64 + j * 32 + (lane & 31);
        if (row < m && col < g.N) {
          float v = acc[i][j][r];
          if constexpr (EPI == EPI_RELU) v = fmaxf(v, 0.f);
          if constexpr (EPI == EPI_SWIGLU) v = silu_f(v) * acc3[i][j][r];
          g.C[(int64_t)(row0 + row) * g.ldc + col] = f32_to_bf16(v);
        }
      }
}

// ---------------------------------------------------------------------------
// Large layers (on average >= GB_BM rows per expert): 256 x 256 output tiles
// (256 x 128 with the SwiGLU epilogue), K staged through LDS 64 at a time,
// eight waves (two per SIMD, so one wave's MFMAs cover the other's LDS waits
// and barriers) of 128 x 64 (SwiGLU: 128 x 32) each.  Per 16-deep k-step a
// wave reads four activation and two (SwiGLU: one and one) weight fragments
// for eight MFMAs.
//   * Operand tiles go from global memory straight into LDS
//     (global_load_lds_dwordx4: each wave-wide load fills 1 KB of LDS in lane
//     order), with no staging registers and no LDS store pass.  A tile row is
//     64 elements = 8 chunks of 16 bytes; chunk c of row R sits at slot
//     R*8 + (c ^ ((R >> 1) & 7)), so the 16 rows a fragment read touches land
//     in 16 different bank groups; each lane loads the chunk that belongs in
//     its slot.
//   * The MFMAs run transposed (weights in operand A), so an accumulator lane
//     holds four consecutive output columns of one row and the epilogue
//     stores them as 8 bytes.
//   * Tiles go in windows of GB_WIN = 8 row tiles.  When there are at least
//     32 column tiles, a multiple of 8, each XCD runs the window's 8 row
//     tiles against every 8th column tile, so a weight tile is fetched by one
//     XCD and read from its L2 by 8 workgroups, and 8 activation tiles are
//     shared by the XCD's 32 CUs.  Otherwise consecutive workgroups take the
//     window's row tiles against one column tile, then the next (with fewer
//     column tiles an XCD's CUs would hold tiles of several windows).
// The same kernel serves the backward of such layers (template arguments):
//   * EPI_RELU_BWD / EPI_SWIGLU_BWD: the first GEMM's products with an
//     epilogue that reads dHid and writes the recomputed hidden activations
//     and the pre-activation gradients.
//   * TBB: weights stored [K][N] (W2 for dHid = dY W2, W1 and W3 for dX),
//     brought into LDS as stored and read into MFMA fragments by the
//     transposing LDS read; A2, B2 add a second operand pair along K.
//   * WGT: per-expert table gradients, both operands [positions][columns]
//     through the transposing read, K over the expert's positions, rows past
//     them read from a zero row.
// ---------------------------------------------------------------------------
constexpr int GB_BM = 256, GB_BK = 64, GB_WIN = 8;
// column tile: 128 with the SwiGLU epilogue (two accumulator sets), 256
// otherwise
template <int EPI> constexpr int gb_bn() {
  return EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD ? 128 : 256;
}

// element offset of chunk c (8 elements) of row r in a swizzled operand tile
__device__ __forceinline__ int gb_slot(int r, int c) { return (r * 8 + (c ^ ((r >> 1) & 7))) * 8; }

// Transposed read of four k values of one weight column from a [k][n] LDS
// tile (BN columns, 16-byte chunks swizzled as chunk ^ 2 (row & 3)).  Within
// each group of 16 lanes, lane j points at row kb + j / 4, columns
// nb + 4 (j % 4) .. +3, and ds_read_b64_tr_b16 hands lane i the values at
// rows kb .. kb + 3 of column nb + i: lane i of group G receives column
// nb(G) + i, rows kb(G) .. kb(G) + 3.
template <int BN>
__device__ __forceinline__ v4i16_t gb_read_tr(const bf16_t* T, int row, int n) {
  const int slot = row * (BN / 8) + ((n >> 3) ^ (2 * (row & 3)));
  typedef v4i16_t __attribute__((address_space(3))) * lds_v4p;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(T + slot * 8 + (n & 7)));
}

template <int EPI, bool TBB, bool WGT>
__global__ __launch_bounds__(512, 1) void grouped_gemm_big_kernel(GemmArgs g) {
  constexpr bool SW = (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD);
  constexpr bool BWD = (EPI == EPI_RELU_BWD || EPI == EPI_SWIGLU_BWD);
  static_assert(!TBB || EPI == EPI_NONE, "weights stored [K][N] only for plain products");
  static_assert(!WGT || TBB, "table gradients read both operands as [K][rows]");
  constexpr int BN = gb_bn<EPI>();
  constexpr int NBJ = BN / 64;   // 1 KB weight blocks each wave loads per slice
  constexpr int WN = BN / 4;     // columns per wave
  constexpr int NJ = WN / 32;    // 32-column MFMA blocks per wave
  constexpr int AT = GB_BM * GB_BK, BT = BN * GB_BK;  // tile elements
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  bf16_t* As = smem;               // [2][AT]
  bf16_t* Bs = As + 2 * AT;        // [2][BT]
  bf16_t* B3s = Bs + 2 * BT;       // [2][BT], SwiGLU only
  __shared__ int s_e, s_row0, s_m, s_ct, s_k0, s_kn;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) {
    // row tiles: of the routed rows (tile map), or WGT: wrows per expert
    const int Q = WGT ? g.E * g.wrows : g.tiles[g.E];
    const int per_win = GB_WIN * g.ncol;
    const int win = blockIdx.x / per_win, within = blockIdx.x % per_win;
    // workgroups go to the XCDs round robin: with at least 32 column tiles,
    // a multiple of 8, XCD x = within % 8 takes the window's row tiles
    // against column tiles x, x + 8, x + 16, ...  At a time its 32 CUs run 8
    // row tiles against 4 column tiles, so each weight tile is fetched into
    // one XCD's L2 and read there by 8 workgroups
    int qw = within % GB_WIN, ct = within / GB_WIN;
    if (g.ncol % 8 == 0 && g.ncol >= 32) {
      const int x = within % 8, j = within / 8;
      qw = j % GB_WIN;
      ct = (j / GB_WIN) * 8 + x;
    }
    const int q = win * GB_WIN + qw;
    if (q < Q) {
      if constexpr (WGT) {
        const int e = q / g.wrows, r = q % g.wrows;
        const int mt = g.wswap ? ct : r;
        s_e = e;
        s_row0 = mt * GB_BM;
        s_m = min(GB_BM, g.M - mt * GB_BM);
        s_k0 = g.offsets[e];
        s_kn = g.offsets[e + 1] - g.offsets[e];
        s_ct = g.wswap ? r : ct;
      } else {
        const int e = expert_of_tile(g.tiles, g.E, q);
        const int row0 = g.offsets[e] + (q - g.tiles[e]) * GB_BM;
        s_e = e;
        s_row0 = row0;
        s_m = min(GB_BM, g.offsets[e + 1] - row0);
        s_k0 = 0;
        s_kn = g.K;
        s_ct = ct;
      }
    } else {
      s_e = -1;
    }
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_e);
  if (e < 0) return;
  const int row0 = __builtin_amdgcn_readfirstlane(s_row0);
  const int m = __builtin_amdgcn_readfirstlane(s_m);
  const int n0 = __builtin_amdgcn_readfirstlane(s_ct) * BN;
  const int kstart = __builtin_amdgcn_readfirstlane(s_k0);
  const int kn = __builtin_amdgcn_readfirstlane(s_kn);

  // Direct loads: wave w fills 1 KB blocks w*4 + j (A, j < 4) and
  // w*NBJ + j (B, B3, j < NBJ); lane l of block b fills slot 64b + l.
  //   K-major tiles (activations; weights stored [N][K]): row (64b + l) / 8,
  //   chunk position l % 8, i.e. source chunk (l % 8) ^ ((row >> 1) & 7).
  //   Weights stored [K][N] (TBB): the tile is [k][n], 32 chunks per k row:
  //   row 2b + l / 32, chunk position l % 32, i.e. source chunk
  //   (l % 32) ^ (2 (row & 3)).
  // Offsets are kept per lane so that a second operand pair can use them.
  // (arrays of a fixed size: the lambdas below capture them, and the host
  // pass of the compiler drops the kernel when a captured array's bound
  // depends on the template argument; unused entries are optimised out)
  //   WGT: both tiles are [k][rows] like the TBB weight tile; the k row of
  //   each load (ar, br) decides between the position's row and the zero row.
  int64_t aoff[4], boff[4];
  int ar[4], br[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (WGT) {
      const int r = 2 * (w * 4 + j) + (lane >> 5);
      const int c = (lane & 31) ^ (2 * (r & 3));
      ar[j] = r;
      aoff[j] = min(row0 + 8 * c, g.M - 8);
    } else {
      const int r = (w * 4 + j) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int p = row0 + min(r, m - 1);
      const int64_t src = g.perm ? (int64_t)(g.perm[p] / g.k) : (int64_t)p;
      ar[j] = 0;
      aoff[j] = src * g.lda + c * 8;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (TBB) {
      const int r = 2 * (w * NBJ + (j < NBJ ? j : 0)) + (lane >> 5);
      const int c = (lane & 31) ^ (2 * (r & 3));
      const int n = min(n0 + 8 * c, g.N - 8);
      br[j] = r;
      boff[j] = WGT ? (int64_t)n : (int64_t)e * g.N * g.K + (int64_t)r * g.N + n;
    } else {
      br[j] = 0;
      const int r = (w * NBJ + (j < NBJ ? j : 0)) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((r >> 1) & 7);
      const int n = min(n0 + r, g.N - 1);
      boff[j] = ((int64_t)e * g.N + n) * g.K + c * 8;
    }
  }
  const int nk = WGT ? (kn + GB_BK - 1) / GB_BK : g.K / GB_BK;
  // slice kt of the K loop: the first pair's slices, then the second's
  auto dma = [&](int kt, int buf) {
    if constexpr (WGT) {
      const int k0 = kt * GB_BK;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = k0 + ar[j];
        const bf16_t* src =
            kk < kn ? g.A + (int64_t)(kstart + kk) * g.lda + aoff[j] : g.zero + aoff[j];
        __builtin_amdgcn_global_load_lds(src, As + buf * AT + (w * 4 + j) * 512, 16, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < NBJ; ++j) {
        const int kk = k0 + br[j];
        const bf16_t* src =
            kk < kn ? g.B + (int64_t)(kstart + kk) * g.N + boff[j] : g.zero + boff[j];
        __builtin_amdgcn_global_load_lds(src, Bs + buf * BT + (w * NBJ + j) * 512, 16, 0, 0);
      }
      return;
    }
    const bool second = kt >= nk;
    const int k0 = (second ? kt - nk : kt) * GB_BK;
    const bf16_t* Ab = second ? g.A2 : g.A;
    const bf16_t* Bb = second ? g.B2 : g.B;
    const int64_t bk = TBB ? (int64_t)k0 * g.N : (int64_t)k0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(Ab + aoff[j] + k0, As + buf * AT + (w * 4 + j) * 512, 16, 0,
                                       0);
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      __builtin_amdgcn_global_load_lds(Bb + boff[j] + bk, Bs + buf * BT + (w * NBJ + j) * 512, 16,
                                       0, 0);
      if constexpr (SW)
        __builtin_amdgcn_global_load_lds(g.B3 + boff[j] + bk, B3s + buf * BT + (w * NBJ + j) * 512,
                                         16, 0, 0);
    }
  };

  const int wm = w >> 2, wn = w & 3;  // wave tile: rows wm*128 .. +128, cols wn*WN .. +WN
  const bool active = wm * 128 < m;
  const int fr = lane & 31, fh = lane >> 5;
  f32x16 acc[4][4], acc3[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
  if constexpr (SW) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc3[i][j] = f32x16{};
  }

  const int nkt = (g.A2 ? 2 : 1) * nk;
  if (nkt > 0) dma(0, 0);  // (an expert without rows: zero gradients)
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    // the next K slice streams into the other buffer while this one is used
    if (kt + 1 < nkt) dma(kt + 1, buf ^ 1);
    // every wave runs the MFMAs (rows past m hold copies of a valid row and are
    // dropped at the store): a branch here would make the compiler keep a
    // second copy of the accumulators
    {
      const bf16_t* Ab = As + buf * AT;
      const bf16_t* Bb = Bs + buf * BT;
      const bf16_t* B3b = B3s + buf * BT;
      // operand fragments one 16-deep k-step ahead of the MFMAs, no further
      bf16x8 af[2][4], bf[2][4], b3f[2][2];
      auto frags = [&](int st, int sl) {
        const int c = 2 * st + fh;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (WGT) {
            // row wm*128 + 32i + lane % 32, k = 16 st + 8 (lane / 32) + 0..7
            const int G = lane >> 4, jj = lane & 15;
            const int mb = wm * 128 + i * 32 + 16 * (G & 1) + 4 * (jj & 3);
            const int kb = st * 16 + 8 * (G >> 1) + (jj >> 2);
            const v4i16_t lo = gb_read_tr<GB_BM>(Ab, kb, mb);
            const v4i16_t hi = gb_read_tr<GB_BM>(Ab, kb + 4, mb);
            af[sl][i] = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          } else {
            af[sl][i] = *reinterpret_cast<const bf16x8*>(Ab + gb_slot(wm * 128 + i * 32 + fr, c));
          }
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          if constexpr (TBB) {
            // column wn*WN + 32j + lane % 32, k = 16 st + 8 (lane / 32) + 0..7
            const int G = lane >> 4, jj = lane & 15;
            const int nb = wn * WN + j * 32 + 16 * (G & 1) + 4 * (jj & 3);
            const int kb = st * 16 + 8 * (G >> 1) + (jj >> 2);
            const v4i16_t lo = gb_read_tr<BN>(Bb, kb, nb);
            const v4i16_t hi = gb_read_tr<BN>(Bb, kb + 4, nb);
            bf[sl][j] = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          } else {
            bf[sl][j] = *reinterpret_cast<const bf16x8*>(Bb + gb_slot(wn * WN + j * 32 + fr, c));
          }
          if constexpr (SW)
            b3f[sl][j] = *reinterpret_cast<const bf16x8*>(B3b + gb_slot(wn * WN + j * 32 + fr, c));
        }
      };
      frags(0, 0);
#pragma unroll
      for (int st = 0; st < GB_BK / 16; ++st) {
        const int sl = st & 1;
        if (st + 1 < GB_BK / 16) frags(st + 1, sl ^ 1);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            acc[i][j] = mfma32(bf[sl][j], af[sl][i], acc[i][j]);
            if constexpr (SW) acc3[i][j] = mfma32(b3f[sl][j], af[sl][i], acc3[i][j]);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the next slice has landed (the barrier waits for the direct loads) and
    // every wave is done with this one
    __syncthreads();
  }

  if (!active) return;
  // register group q of acc[i][j] holds columns wn*WN + 32j + 8q + 4(lane/32) .. +3
  // of row wm*128 + 32i + lane%32
  const int q4 = fh * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wm * 128 + 32 * i + fr;
    if (row >= m) continue;
    const int64_t roff = (WGT ? (int64_t)e * g.M * g.N : 0) + (int64_t)(row0 + row) * g.ldc;
    bf16_t* crow = g.C + roff;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * WN + 32 * j + 8 * q + q4;
        const bool full = col + 3 < g.N;
        float v[4], v2[4], v3[4];
        if constexpr (BWD) {
          // this lane's dHid values; it overwrites them below
          float dh[4];
          if (full) {
            const uint2 u = *reinterpret_cast<const uint2*>(g.C2 + roff + col);
            dh[0] = __uint_as_float(u.x << 16);
            dh[1] = __uint_as_float(u.x & 0xffff0000u);
            dh[2] = __uint_as_float(u.y << 16);
            dh[3] = __uint_as_float(u.y & 0xffff0000u);
          } else {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              dh[r] = col + r < g.N ? bf16_to_f32(g.C2[roff + col + r]) : 0.f;
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float a = acc[i][j][4 * q + r];
            if constexpr (EPI == EPI_RELU_BWD) {
              v[r] = fmaxf(a, 0.f);
              v2[r] = a > 0.f ? dh[r] : 0.f;
              v3[r] = 0.f;
            } else {
              const float b = acc3[i][j][4 * q + r];
              const float sg = 1.0f / (1.0f + expf(-a));
              const float sl = a * sg;
              v[r] = sl * b;
              v2[r] = dh[r] * b * sg * (1.0f + a * (1.0f - sg));
              v3[r] = dh[r] * sl;
            }
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = acc[i][j][4 * q + r];
            if constexpr (EPI == EPI_RELU) x = fmaxf(x, 0.f);
            if constexpr (EPI == EPI_SWIGLU) x = silu_f(x) * acc3[i][j][4 * q + r];
            v[r] = x;
          }
        }
        if (full) {
          *reinterpret_cast<uint2*>(crow + col) = uint2{cvt_pk_bf16(v[0], v[1]), cvt_pk_bf16(v[2], v[3])};
          if constexpr (BWD)
            *reinterpret_cast<uint2*>(g.C2 + roff + col) =
                uint2{cvt_pk_bf16(v2[0], v2[1]), cvt_pk_bf16(v2[2], v2[3])};
          if constexpr (EPI == EPI_SWIGLU_BWD)
            *reinterpret_cast<uint2*>(g.C3 + roff + col) =
                uint2{cvt_pk_bf16(v3[0], v3[1]), cvt_pk_bf16(v3[2], v3[3])};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (col + r < g.N) {
              crow[col + r] = f32_to_bf16(v[r]);
              if constexpr (BWD) g.C2[roff + col + r] = f32_to_bf16(v2[r]);
              if constexpr (EPI == EPI_SWIGLU_BWD) g.C3[roff + col + r] = f32_to_bf16(v3[r]);
            }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// fp32 path: one thread per output element.
// ---------------------------------------------------------------------------
// sum_c a[c] b[c] in c order, 16-byte loads when both rows allow them
__device__ __forceinline__ float dot_f32(const float* a, const float* b, int n) {
  float s = 0.f;
  int c = 0;
  if (((n | (int)((uintptr_t)a | (uintptr_t)b)) & 3) == 0 &&
      (((uintptr_t)a | (uintptr_t)b) & 15) == 0) {
    for (; c < n; c += 4) {
      const float4 x = *reinterpret_cast<const float4*>(a + c);
      const float4 y = *reinterpret_cast<const float4*>(b + c);
      s = fmaf(x.x, y.x, s);
      s = fmaf(x.y, y.y, s);
      s = fmaf(x.z, y.z, s);
      s = fmaf(x.w, y.w, s);
    }
  }
  for (; c < n; ++c) s = fmaf(a[c], b[c], s);
  return s;
}

__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int p) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(256) void ffn1_f32_kernel(FfnArgs a, int swiglu) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.A * a.h) return;
  const int p = (int)(i / a.h), j = (int)(i % a.h);
  const int e = expert_of_row(a.offsets, a.E, p);
  const int64_t src = a.perm ? (int64_t)(a.perm[p] / a.k) : (int64_t)p;
  const float* xr = (const float*)a.x + src * a.d;
  const float* w1 = (const float*)a.w1 + ((int64_t)e * a.h + j) * a.d;
  const float* w3 = swiglu ? (const float*)a.w3 + ((int64_t)e * a.h + j) * a.d : w1;
  const float s = dot_f32(xr, w1, a.d);
  float v;
  if (swiglu) {
    const float u = dot_f32(xr, w3, a.d);
    v = silu_f(s) * u;
  } else {
    v = fmaxf(s, 0.f);
  }
  ((float*)a.hid)[i] = v;
}

__global__ __launch_bounds__(256) void ffn2_f32_kernel(FfnArgs a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= a.A * a.d) return;
  const int p = (int)(i / a.d), n = (int)(i % a.d);
  const int e = expert_of_row(a.offsets, a.E, p);
  const float* hr = (const float*)a.hid + (int64_t)p * a.h;
  const float* w2 = (const float*)a.w2 + ((int64_t)e * a.d + n) * a.h;
  ((float*)a.y_sorted)[i] = dot_f32(hr, w2, a.h);
}

// The large-tile kernel pays off once the experts average a full tile of rows.
static bool big_tiles(int64_t A, int E) { return A >= (int64_t)GB_BM * E; }

int ffn_tile_rows(bool bf16, int d, int h, int swiglu, int64_t A, int E) {
  if (!bf16) return 1;
  if (fused_ffn_supported(d, h, swiglu)) return 0;  // finds its tiles from the offsets
  return big_tiles(A, E) ? GB_BM : GM_BM;
}

template <int EPI, bool TBB = false, bool WGT = false>
static hipError_t launch_big(const GemmArgs& g, int64_t qmax, hipStream_t s) {
  constexpr bool SW = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_BWD;
  constexpr size_t lds = sizeof(bf16_t) * (size_t)GB_BK * 2 * (GB_BM + gb_bn<EPI>() * (SW ? 2 : 1));
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t err = hipFuncSetAttribute((const void*)grouped_gemm_big_kernel<EPI, TBB, WGT>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_done = true;
  }
  const int64_t wins = (qmax + GB_WIN - 1) / GB_WIN;
  hipLaunchKernelGGL((grouped_gemm_big_kernel<EPI, TBB, WGT>),
                     dim3((unsigned)(wins * GB_WIN * g.ncol)), dim3(512), lds, s, g);
  return hipGetLastError();
}

hipError_t launch_expert_ffn(const FfnArgs& a, bool bf16, int swiglu, hipStream_t s) {
  if (a.A == 0) return hipSuccess;
  if (!bf16) {
    hipLaunchKernelGGL(ffn1_f32_kernel, dim3((unsigned)((a.A * a.h + 255) / 256)), dim3(256), 0, s,
                       a, swiglu);
    hipLaunchKernelGGL(ffn2_f32_kernel, dim3((unsigned)((a.A * a.d + 255) / 256)), dim3(256), 0, s,
                       a);
    return hipGetLastError();
  }
  if (fused_ffn_supported(a.d, a.h, swiglu)) return launch_fused_ffn(a, s);
  const bool big = big_tiles(a.A, a.E);
  const int bm = big ? GB_BM : GM_BM;
  const int bn1 = big ? (swiglu ? gb_bn<EPI_SWIGLU>() : gb_bn<EPI_RELU>()) : GM_BN;
  const int bn2 = big ? gb_bn<EPI_NONE>() : GM_BN;
  // upper bound of tiles: each non-empty expert adds at most one partial tile
  const int64_t qmax = (a.A + bm - 1) / bm + a.E;
  GemmArgs g1;
  g1.A = (const bf16_t*)a.x;
  g1.lda = a.d;
  g1.perm = a.perm;
  g1.k = a.k;
  g1.B = (const bf16_t*)a.w1;
  g1.B3 = (const bf16_t*)a.w3;
  g1.N = a.h;
  g1.K = a.d;
  g1.offsets = a.offsets;
  g1.tiles = a.tiles;
  g1.E = a.E;
  g1.C = (bf16_t*)a.hid;
  g1.ldc = a.h;
  g1.ncol = (a.h + bn1 - 1) / bn1;
  GemmArgs g2 = g1;
  g2.A = (const bf16_t*)a.hid;
  g2.lda = a.h;
  g2.perm = nullptr;
  g2.B = (const bf16_t*)a.w2;
  g2.B3 = nullptr;
  g2.N = a.d;
  g2.K = a.h;
  g2.C = (bf16_t*)a.y_sorted;
  g2.ldc = a.d;
  g2.ncol = (a.d + bn2 - 1) / bn2;
  if (big) {
    hipError_t err = swiglu ? launch_big<EPI_SWIGLU>(g1, qmax, s) : launch_big<EPI_RELU>(g1, qmax, s);
    if (err != hipSuccess) return err;
    return launch_big<EPI_NONE>(g2, qmax, s);
  }
  if (swiglu)
    hipLaunchKernelGGL(grouped_gemm_kernel<EPI_SWIGLU>, dim3((unsigned)(qmax * g1.ncol)), dim3(256),
                       0, s, g1);
  else
    hipLaunchKernelGGL(grouped_gemm_kernel<EPI_RELU>, dim3((unsigned)(qmax * g1.ncol)), dim3(256), 0,
                       s, g1);
  hipLaunchKernelGGL(grouped_gemm_kernel<EPI_NONE>, dim3((unsigned)(qmax * g2.ncol)), dim3(256), 0,
                     s, g2);
  return hipGetLastError();
}

bool bw_hidden_big_tiles(bool bf16, int64_t A, int E) { return bf16 && big_tiles(A, E); }
int bw_hidden_big_rows() { return GB_BM; }

// The backward's hidden layer on the large-tile kernel: the forward's first
// GEMM over the routed rows (X W1_e^T, and X W3_e^T with SwiGLU), with an
// epilogue that takes dHid from d1 and leaves the recomputed activations in
// hid, dP or dA in d1 and dB in d3.
hipError_t launch_bw_hidden_big(const BwHiddenArgs& a, bool swiglu, hipStream_t s) {
  if (a.A == 0) return hipSuccess;
  const int bn = swiglu ? gb_bn<EPI_SWIGLU_BWD>() : gb_bn<EPI_RELU_BWD>();
  GemmArgs g;
  g.A = (const bf16_t*)a.xs;
  g.lda = a.d;
  g.perm = nullptr;
  g.k = 1;
  g.B = (const bf16_t*)a.w1;
  g.B3 = (const bf16_t*)a.w3;
  g.N = a.h;
  g.K = a.d;
  g.offsets = a.offsets;
  g.tiles = a.tiles;
  g.E = a.E;
  g.C = (bf16_t*)a.hid;
  g.ldc = a.h;
  g.ncol = (a.h + bn - 1) / bn;
  g.C2 = (bf16_t*)a.d1;
  g.C3 = (bf16_t*)a.d3;
  const int64_t qmax = (a.A + GB_BM - 1) / GB_BM + a.E;
  return swiglu ? launch_big<EPI_SWIGLU_BWD>(g, qmax, s) : launch_big<EPI_RELU_BWD>(g, qmax, s);
}

// A plain product of the backward on the large tiles: c = a b_e (+ a2 b2_e)
// per routed row, with the tables stored [E][K][N] (read across their rows
// through the transposed LDS reads).
hipError_t launch_bw_big_product(const BwBigProduct& p, hipStream_t s) {
  if (p.A == 0) return hipSuccess;
  if (p.N % 8 != 0 || p.K % GB_BK != 0) return hipErrorInvalidValue;
  GemmArgs g;
  g.A = (const bf16_t*)p.a;
  g.lda = p.K;
  g.perm = nullptr;
  g.k = 1;
  g.B = (const bf16_t*)p.b;
  g.B3 = nullptr;
  g.N = p.N;
  g.K = p.K;
  g.offsets = p.offsets;
  g.tiles = p.tiles;
  g.E = p.E;
  g.C = (bf16_t*)p.c;
  g.ldc = p.N;
  g.ncol = (p.N + gb_bn<EPI_NONE>() - 1) / gb_bn<EPI_NONE>();
  g.A2 = (const bf16_t*)p.a2;
  g.B2 = (const bf16_t*)p.b2;
  const int64_t qmax = (p.A + GB_BM - 1) / GB_BM + p.E;
  return launch_big<EPI_NONE, true>(g, qmax, s);
}

// Per-expert table gradients on the large tiles: c_e [M][N] = a_e^T b_e
// over the positions of expert e (a [A][M], b [A][N] bf16 in expert order,
// c [E][M][N] bf16); zero: max(M, N) bf16 zeros.
hipError_t launch_bw_big_wgrad(const BwBigWgrad& p, hipStream_t s) {
  if (p.E == 0) return hipSuccess;
  if (p.M % 8 != 0 || p.N % 8 != 0) return hipErrorInvalidValue;
  GemmArgs g;
  g.A = (const bf16_t*)p.a;
  g.lda = p.M;
  g.perm = nullptr;
  g.k = 1;
  g.B = (const bf16_t*)p.b;
  g.B3 = nullptr;
  g.N = p.N;
  g.K = 0;
  g.offsets = p.offsets;
  g.tiles = nullptr;
  g.E = p.E;
  g.C = (bf16_t*)p.c;
  g.ldc = p.N;
  // an expert's output tiles in the enumeration: its row tiles against its
  // column tiles, or the other way round when only the row tiles are enough
  // for the XCD-grouped order
  const int mt = (p.M + GB_BM - 1) / GB_BM;
  const int nt = (p.N + gb_bn<EPI_NONE>() - 1) / gb_bn<EPI_NONE>();
  g.wswap = nt < 32 && mt >= 32 && mt % 8 == 0;
  g.wrows = g.wswap ? nt : mt;
  g.ncol = g.wswap ? mt : nt;
  g.M = p.M;
  g.zero = (const bf16_t*)p.zero;
  return launch_big<EPI_NONE, true, true>(g, (int64_t)p.E * g.wrows, s);
}

}  // namespace moe
