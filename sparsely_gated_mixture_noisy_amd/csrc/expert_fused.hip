// Fused ReLU expert FFN for d_model = 512: y = max(x W1^T, 0) W2^T per routed
// row, the hidden activation never leaving the chip.
//
// The expert is the one-hidden-layer ReLU FFN of the MoE lesson page
// ("MoE:稀疏门控混合专家", section 二: 512 -> 1024 -> 512).  With k*b/n rows
// per expert (paper card, section 瓶颈: about 128 at 8192 tokens, 256 experts,
// k = 4) the expert stage is bound by streaming the expert tables from HBM,
// not by MFMA, so the kernel is organised to read each table byte once:
//
//   * one workgroup = one tile of at most 96 rows of one expert (an expert
//     with m rows gets ceil(m/96) tiles, its 32-row blocks spread evenly
//     over them, whole blocks first); the tiles of an
//     expert have consecutive ids that land on one XCD and are dispatched
//     together, so they share the weight stream through that XCD's L2;
//   * the tile's gathered input rows sit in LDS (96 x 512 bf16);
//   * eight waves, two per SIMD, so that one wave's MFMAs cover the other's
//     waits on memory, LDS and barriers;
//   * the hidden layer is produced 256 units at a time: each wave computes
//     S = relu(X W1[32 units]^T) for the tile's rows (v_mfma_f32_32x32x16_bf16,
//     W1 fragments streamed from global memory into a register ring), writes
//     it as bf16 to LDS, then every wave accumulates Y[:, its 64 columns] +=
//     S W2[cols, 256 units]^T with W2 fragments streamed the same way; only
//     the 32-row blocks that hold rows of the tile go through the MFMAs;
//   * Y (up to 96 x 512 fp32) stays in registers across the hidden chunks and
//     is written once, as bf16, through LDS for coalesced 16-byte stores;
//   * the expert tables can be repacked once (moe_pack_experts) into the
//     exact order the waves consume their 16-byte fragments, so that every
//     wave-wide load reads 1 KB of contiguous memory instead of 32-byte pieces
//     of 32 rows.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int FZ_MT = 3;      // 32-row blocks per tile (rows per tile: 32 * FZ_MT)
constexpr int FZ_M = 32 * FZ_MT;
constexpr int FZ_H = 256;     // hidden units per chunk
constexpr int FZ_WAVES = 8;
constexpr int FZ_THREADS = 64 * FZ_WAVES;
constexpr int FZ_D = 512;     // d_model handled by this kernel
constexpr int FZ_RING = 8;    // weight fragments in flight per wave

struct FusedArgs {
  const bf16_t* x;
  const int32_t* perm;  // null: row p is x[p]
  int k;
  const int32_t* offsets;  // [E+1] routing offsets: expert e holds positions
                           // offsets[e] .. offsets[e+1]-1
  int E, h;
  const bf16_t* w1;      // [E][h][D]   (unpacked)
  const bf16_t* w2;      // [E][D][h]   (unpacked)
  const bf16_t* wp;      // packed tables, or null
  bf16_t* y;             // [A][D]
};

// The weight stream of one wave.  For hidden chunk hc (FZ_H units), wave w
// consumes NE 16-byte fragments per lane:
//   n <  N1: W1 fragments, k-step n, of the wave's U1 = 32 hidden units
//            [hc*FZ_H + 32w, +32);
//   n >= N1: W2 fragments, k-step (n-N1)/NT2, 32-column block (n-N1)%NT2 of
//            the wave's C2 = D/8 output columns [w*C2, +C2).
// src() gives the element offset of a fragment inside expert e's unpacked
// tables (table 0: W1 [h][D], table 1: W2 [D][h]); the packed layout stores
// the fragments contiguously in consumption order:
// [e][hc][w][n][lane][8 elements].
template <int D>
struct Stream {
  static constexpr int U1 = FZ_H / FZ_WAVES;   // hidden units per wave per chunk
  static constexpr int KS1 = D / 16;           // first-layer k-steps
  static constexpr int C2 = D / FZ_WAVES;      // output columns per wave
  static constexpr int NT2 = C2 / 32;          // 32-wide output blocks per wave
  static constexpr int KS2 = FZ_H / 16;        // second-layer k-steps per chunk
  static constexpr int N1 = KS1, NE = N1 + NT2 * KS2;
  static_assert(U1 == 32, "one 32-unit block per wave");
  static __host__ __device__ inline int64_t src(int h, int hc, int w, int n, int lane,
                                                int* table) {
    const int fr = lane & 31, fk = (lane >> 5) * 8;
    if (n < N1) {
      *table = 0;
      return (int64_t)(hc * FZ_H + w * U1 + fr) * D + n * 16 + fk;
    }
    const int mm = n - N1, ks = mm / NT2, j = mm % NT2;
    *table = 1;
    return (int64_t)(w * C2 + j * 32 + fr) * h + hc * FZ_H + ks * 16 + fk;
  }
  static __host__ __device__ inline int64_t packed(int h, int e, int hc, int w, int n, int lane) {
    const int nch = h / FZ_H;
    return ((((int64_t)e * nch + hc) * FZ_WAVES + w) * NE + n) * 512 + lane * 8;
  }
};

// Weight fragment n of hidden chunk hc of expert e for the calling lane of
// its wave (see Stream).
template <int D, bool PACKED>
__device__ __forceinline__ u32x4 fused_frag(const FusedArgs& a, int e, int hc, int n) {
  using S = Stream<D>;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if constexpr (PACKED) {
    return *reinterpret_cast<const u32x4*>(a.wp + S::packed(a.h, e, hc, w, n, lane));
  } else {
    int t;
    const int64_t o = S::src(a.h, hc, w, n, lane, &t);
    const bf16_t* base = t == 0 ? a.w1 + (int64_t)e * a.h * D : a.w2 + (int64_t)e * D * a.h;
    return *reinterpret_cast<const u32x4*>(base + o);
  }
}

// One tile of m <= 32*MB rows of expert e, rows p0 .. p0+m-1 of the routed
// order (input row s_src[r]).  Both layers run transposed on the MFMA: the
// weight fragment is operand A and the activation fragment operand B, so an
// accumulator lane holds four consecutive hidden units (first layer) or
// output columns (second layer) of one row, which go to LDS as one 8-byte
// store of two packed bf16 pairs.
template <int D, int MB, bool PACKED>
__device__ __forceinline__ void fused_tile(const FusedArgs& a, int e, int p0, int m,
                                           bf16_t* Xs, bf16_t* Ss, const int* s_src,
                                           u32x4 (&ring)[FZ_RING]) {
  using S = Stream<D>;
  constexpr int XLD = D + 8;     // LDS row stride of the input tile (elements)
  constexpr int SLD = FZ_H + 8;  // LDS row stride of the hidden tile
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int XCH = 32 * MB * CPR;                             // input chunks of the tile
  constexpr int XPT = (XCH + FZ_THREADS - 1) / FZ_THREADS;       // per thread
  constexpr int N1 = S::N1, NE = S::NE, NT2 = S::NT2, RING = FZ_RING;
  static_assert(NE % RING == 0 && N1 % RING == 0, "stream must be a multiple of the ring");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 31, fk = (lane >> 5) * 8, q4 = (lane >> 5) * 4;
  const int nchunks = a.h / FZ_H;
  auto frag = [&](int hc, int n) -> u32x4 { return fused_frag<D, PACKED>(a, e, hc, n); };

  // gathered input rows (rows past m are zero); the ring already holds the
  // requests for the first RING weight fragments
  u32x4 xv[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = tid + i * FZ_THREADS, r = c / CPR, cc = (c % CPR) * 8;
    xv[i] = (c < XCH && r < m) ? *reinterpret_cast<const u32x4*>(a.x + (int64_t)s_src[r] * D + cc)
                               : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = tid + i * FZ_THREADS, r = c / CPR, cc = (c % CPR) * 8;
    if (c < XCH) *reinterpret_cast<u32x4*>(Xs + r * XLD + cc) = xv[i];
  }

  f32x16 acc[MB][NT2];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NT2; ++j) acc[i][j] = f32x16{};

  __syncthreads();
  for (int hc = 0; hc < nchunks; ++hc) {
    const bool more = hc + 1 < nchunks;
    // consume entry n of this chunk's stream and refill its ring slot.  Every
    // take issues a load: after the last chunk the refills all read this
    // chunk's first fragment again (a cache hit), so that no load hangs on a
    // branch and the compiler's wait counts stay at the ring's depth instead
    // of draining it at each chunk's end.
    auto take = [&](int n) -> bf16x8 {
      const bf16x8 v = __builtin_bit_cast(bf16x8, ring[n % RING]);
      const int nn = n + RING;
      if (nn < NE) ring[n % RING] = frag(hc, nn);
      else ring[n % RING] = frag(more ? hc + 1 : hc, more ? nn - NE : 0);
      return v;
    };
    // ---- first layer: S^T[32w .. +32 units][rows] = W1[units] X^T ----
    f32x16 sa[MB];
    bf16x8 xa[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      sa[i] = f32x16{};
      xa[i] = *reinterpret_cast<const bf16x8*>(Xs + (32 * i + fr) * XLD + fk);
    }
#pragma unroll
    for (int ks = 0; ks < S::KS1; ++ks) {
      const bf16x8 b = take(ks);
      bf16x8 av[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i) av[i] = xa[i];
      if (ks + 1 < S::KS1) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
          xa[i] = *reinterpret_cast<const bf16x8*>(Xs + (32 * i + fr) * XLD + (ks + 1) * 16 + fk);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) sa[i] = mfma32(b, av[i], sa[i]);
      // keep each k-step's refill where it is issued: left free, the
      // scheduler sinks the refills next to their uses and the ring drains
      // (three row blocks have no registers to spare for it and stay free)
      __builtin_amdgcn_sched_barrier(0);
    }
    // relu -> bf16 -> S[row][unit]: register group g holds units
    // 8g + q4 .. +3 of row 32i + fr
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t lo = cvt_pk_bf16(fmaxf(sa[i][4 * g], 0.f), fmaxf(sa[i][4 * g + 1], 0.f));
        const uint32_t hi = cvt_pk_bf16(fmaxf(sa[i][4 * g + 2], 0.f), fmaxf(sa[i][4 * g + 3], 0.f));
        *reinterpret_cast<uint2*>(Ss + (32 * i + fr) * SLD + w * S::U1 + 8 * g + q4) =
            uint2{lo, hi};
      }
    __syncthreads();
    // ---- second layer: Y^T[w*C2 .. +C2 cols][rows] += W2[cols, units] S^T ----
    bf16x8 sv[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) sv[i] = *reinterpret_cast<const bf16x8*>(Ss + (32 * i + fr) * SLD + fk);
#pragma unroll
    for (int ks = 0; ks < S::KS2; ++ks) {
      bf16x8 b[NT2];
#pragma unroll
      for (int j = 0; j < NT2; ++j) b[j] = take(N1 + ks * NT2 + j);
      bf16x8 av[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i) av[i] = sv[i];
      if (ks + 1 < S::KS2) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
          sv[i] = *reinterpret_cast<const bf16x8*>(Ss + (32 * i + fr) * SLD + (ks + 1) * 16 + fk);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NT2; ++j) acc[i][j] = mfma32(b[j], av[i], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
  }

  // Y -> bf16 -> LDS (reusing the input tile) -> coalesced stores; register
  // group g of acc[i][j] holds columns w*C2 + 32j + 8g + q4 .. +3 of row 32i + fr
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NT2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t lo = cvt_pk_bf16(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
        const uint32_t hi = cvt_pk_bf16(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
        *reinterpret_cast<uint2*>(Xs + (32 * i + fr) * XLD + w * S::C2 + 32 * j + 8 * g + q4) =
            uint2{lo, hi};
      }
  __syncthreads();
  // streaming stores: the rows are read once, by the combine
  for (int c = tid; c < m * CPR; c += FZ_THREADS) {
    const int r = c / CPR, cc = (c % CPR) * 8;
    __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(Xs + r * XLD + cc),
                                reinterpret_cast<u32x4*>(a.y + (int64_t)(p0 + r) * D + cc));
  }
}

template <int D, int MT, bool PACKED>
__global__ __launch_bounds__(FZ_THREADS, 1) void ffn_relu_fused_kernel(FusedArgs a) {
  constexpr int M = 32 * MT;     // rows per tile at most
  constexpr int XLD = D + 8;
  static_assert(MT == 3, "the tile body is instantiated for 1 .. 3 row blocks");
  extern __shared__ __attribute__((aligned(16))) bf16_t lds[];
  bf16_t* Xs = lds;
  bf16_t* Ss = lds + M * XLD;
  __shared__ int s_info[3];
  __shared__ int s_src[M];

  const int tid = threadIdx.x;
  // This workgroup's tile, found from the offsets: expert e holds
  // ceil(m_e / M) tiles (m_e its rows), numbered in expert order, its 32-row
  // blocks split over them by tile_rows.  Workgroup b takes tile
  // (b % 8) * ceil(Q / 8) + b / 8 of the Q tiles, so that the tiles of an
  // expert run on one XCD (workgroups go to the XCDs round-robin).
  {
    const int per = (a.E + FZ_THREADS - 1) / FZ_THREADS;  // experts per thread
    const int e0 = min(a.E, tid * per), e1 = min(a.E, e0 + per);
    int nt = 0;
    for (int e = e0; e < e1; ++e) nt += (a.offsets[e + 1] - a.offsets[e] + M - 1) / M;
    int Q;
    int run = block_excl_scan<FZ_THREADS>(nt, &Q);
    const int perx = (Q + 7) / 8;
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int q = xcd * perx + slot;
    if (tid == 0) s_info[0] = -1;
    __syncthreads();
    if (slot < perx && q < Q && q >= run && q < run + nt) {
      for (int e = e0; e < e1; ++e) {
        const int o = a.offsets[e], m = a.offsets[e + 1] - o, n = (m + M - 1) / M;
        if (q < run + n) {
          int first, rows;
          tile_rows(m, n, q - run, &first, &rows);
          s_info[0] = e;
          s_info[1] = o + first;
          s_info[2] = rows;
          break;
        }
        run += n;
      }
    }
  }
  __syncthreads();
  const int e = __builtin_amdgcn_readfirstlane(s_info[0]);
  if (e < 0) return;
  const int p0 = __builtin_amdgcn_readfirstlane(s_info[1]);
  const int m = __builtin_amdgcn_readfirstlane(s_info[2]);
  // A ring of FZ_RING registers keeps that many weight loads in flight
  // without draining between the two layers or between chunks: consuming
  // entry n issues entry n + FZ_RING (of this chunk or the next one).  Its
  // first requests go out before the input rows' gather.
  u32x4 ring[FZ_RING];
#pragma unroll
  for (int i = 0; i < FZ_RING; ++i) ring[i] = fused_frag<D, PACKED>(a, e, 0, i);
  if (tid < M) {
    const int p = p0 + min(tid, m - 1);
    s_src[tid] = a.perm ? a.perm[p] / a.k : p;
  }
  __syncthreads();
  // only the 32-row blocks that hold rows run through the MFMAs
  const int mb = (m + 31) / 32;
  if (mb >= 3)
    fused_tile<D, 3, PACKED>(a, e, p0, m, Xs, Ss, s_src, ring);
  else if (mb == 2)
    fused_tile<D, 2, PACKED>(a, e, p0, m, Xs, Ss, s_src, ring);
  else
    fused_tile<D, 1, PACKED>(a, e, p0, m, Xs, Ss, s_src, ring);
}

bool fused_ffn_supported(int d, int h, int swiglu) {
  return !swiglu && d == FZ_D && h % FZ_H == 0;
}

size_t fused_packed_bytes(int E, int d, int h) {
  return sizeof(bf16_t) * 2 * (size_t)E * d * h;
}

// packed[e][hc][w][n][lane] <- the fragment Stream::src names, 16 bytes a thread
template <int D>
__global__ __launch_bounds__(256) void pack_experts_kernel(const bf16_t* w1, const bf16_t* w2,
                                                           int E, int h, bf16_t* out) {
  using S = Stream<D>;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // fragment-lane index
  const int nch = h / FZ_H;
  const int64_t total = (int64_t)E * nch * FZ_WAVES * S::NE * 64;
  if (i >= total) return;
  const int lane = (int)(i % 64);
  int64_t r = i / 64;
  const int n = (int)(r % S::NE);
  r /= S::NE;
  const int w = (int)(r % FZ_WAVES);
  r /= FZ_WAVES;
  const int hc = (int)(r % nch);
  const int e = (int)(r / nch);
  int t;
  const int64_t o = S::src(h, hc, w, n, lane, &t);
  const bf16_t* src = (t == 0 ? w1 : w2) + (int64_t)e * h * D + o;
  *reinterpret_cast<u32x4*>(out + S::packed(h, e, hc, w, n, lane)) =
      *reinterpret_cast<const u32x4*>(src);
}

hipError_t launch_pack_experts(const void* w1, const void* w2, int E, int d, int h, void* out,
                               hipStream_t s) {
  const int64_t total = (int64_t)E * (h / FZ_H) * FZ_WAVES * Stream<FZ_D>::NE * 64;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(pack_experts_kernel<FZ_D>, dim3((unsigned)((total + 255) / 256)), dim3(256),
                     0, s, (const bf16_t*)w1, (const bf16_t*)w2, E, h, (bf16_t*)out);
  return hipGetLastError();
}

template <bool PACKED>
static hipError_t launch_fused_t(const FusedArgs& a, int64_t A, hipStream_t s) {
  constexpr size_t lds = sizeof(bf16_t) * (size_t)FZ_M * ((FZ_D + 8) + (FZ_H + 8));
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t err = hipFuncSetAttribute((const void*)ffn_relu_fused_kernel<FZ_D, FZ_MT, PACKED>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_done = true;
  }
  // upper bound of tiles, rounded to whole XCD rows
  int64_t qmax = (A + FZ_M - 1) / FZ_M + a.E;
  qmax = (qmax + 7) / 8 * 8;
  hipLaunchKernelGGL((ffn_relu_fused_kernel<FZ_D, FZ_MT, PACKED>), dim3((unsigned)qmax),
                     dim3(FZ_THREADS), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_fused_ffn(const FfnArgs& f, hipStream_t s) {
  FusedArgs a;
  a.x = (const bf16_t*)f.x;
  a.perm = f.perm;
  a.k = f.k;
  a.offsets = f.offsets;
  a.E = f.E;
  a.h = f.h;
  a.w1 = (const bf16_t*)f.w1;
  a.w2 = (const bf16_t*)f.w2;
  a.wp = (const bf16_t*)f.wpacked;
  a.y = (bf16_t*)f.y_sorted;
  return a.wp ? launch_fused_t<true>(a, f.A, s) : launch_fused_t<false>(a, f.A, s);
}

}  // namespace moe
