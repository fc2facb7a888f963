// The backward's hidden layer for the ReLU experts at d_model 512, with the
// expert tables streamed once per tile like the forward's fused kernel.
//
// The backward of y = relu(x W1^T) W2^T (the expert of the MoE lesson page,
// "MoE:稀疏门控混合专家", section 二) needs, for every routed row, the
// hidden activation Hid = relu(a), a = x W1^T (for dW2 = dY^T Hid), and the
// gradient of the pre-activation dP = (dY W2) * [a > 0] (for dW1 = dP^T X
// and dX = dP W1).  Both are products of one row with a whole table, so at
// k*b/n rows per expert (paper card, section 瓶颈) they are bound by reading
// the two tables, and this kernel reads each table byte once per tile:
//
//   * one workgroup = one tile of at most 96 rows of one expert, found from
//     the routing offsets as the forward's fused kernel finds its tiles (its
//     32-row blocks spread evenly over the expert's tiles);
//     the tiles of an expert run on one XCD together and share the table
//     stream through its L2;
//   * the tile gathers its routed rows itself (x, and dy times the slot's
//     gate) and also writes them out in expert order for the table
//     gradients;
//   * phase A: the tile's x rows sit in LDS; for each chunk of 256 hidden
//     units, wave w computes a^T for its 32 units (v_mfma_f32_32x32x16_bf16,
//     W1 fragment as operand A, streamed through a register ring), writes
//     Hid = relu(a) as bf16 and keeps the signs a > 0 as one bit per element
//     in LDS;
//   * phase B: the tile's dy rows replace the x rows; wave w computes
//     (dY W2)^T for the same units and rows, with W2 as operand A: its
//     16-row by 32-unit pieces stream through the same register ring, go to a
//     per-wave LDS slot as loaded (units contiguous) and come back in operand
//     order through gfx950's transposing LDS read; dP is written with the
//     phase-A sign applied.
//   * both results leave through two LDS staging tiles (32 rows x 256 units,
//     used in turn), so that every row's 512 bytes of a chunk are written as
//     whole 16-byte pieces of contiguous rows.
//
// The accumulators of both phases have the same layout (lane l: row l % 32
// of each 32-row block, four consecutive units per register group), so the
// sign bits of an element stay with the lane that produces it.
#include "moe_device.h"
#include "moe_kernels.h"

namespace moe {

constexpr int BH_D = 512;          // d_model handled by this kernel
constexpr int BH_MB = 3;           // 32-row blocks per tile at most
constexpr int BH_M = 32 * BH_MB;   // rows per tile at most
constexpr int BH_H = 256;          // hidden units per chunk
constexpr int BH_WAVES = 8;
constexpr int BH_THREADS = 64 * BH_WAVES;
constexpr int BH_RING = 8;         // table loads in flight per wave (a divisor of BH_KS)
constexpr int BH_MAXCH = 4;        // chunks at most (d_hidden <= 1024): sign bits in LDS
constexpr int BH_KS = BH_D / 16;   // k-steps per chunk, both phases
static_assert(BH_KS % BH_RING == 0, "every chunk starts at ring slot 0");
constexpr int BH_XLD = BH_D + 8;   // LDS row stride of the row tile (elements)
constexpr int BH_SLD = BH_H + 8;   // row stride of the output staging tile (elements)
// Fragments per (expert, chunk, wave) in the forward's packed tables
// (pack_experts_kernel): the wave's BH_KS W1 fragments come first, in k-step
// order, followed by its second-layer fragments.
constexpr int BH_PACK_NE = BH_KS + (BH_D / BH_WAVES / 32) * (BH_H / 16);

// LDS: the row tile, one 16 x 32 slot per wave, the sign bits, two staging tiles
size_t bw_hidden_fused_lds() {
  return sizeof(bf16_t) * ((size_t)BH_M * BH_XLD + (size_t)BH_WAVES * 512) +
         sizeof(uint64_t) * (size_t)BH_MAXCH * BH_WAVES * 64 + sizeof(bf16_t) * 2 * 32 * BH_SLD;
}

bool bw_hidden_fused_supported(bool bf16, int d, int h, bool swiglu) {
  return bf16 && !swiglu && d == BH_D && h % BH_H == 0 && h / BH_H <= BH_MAXCH && h > 0;
}

int64_t bw_hidden_fused_grid(int64_t A, int E) {
  const int64_t q = (A + BH_M - 1) / BH_M + E;  // tiles at most
  return (q + 7) / 8 * 8;
}

// Operand-A fragment of 32 units x 16 k values from a wave's LDS slot that
// holds W2[k0 + c][u0 + u] at element 32 c + u (c < 16, u < 32): lane l gets
// unit l % 32, k values 8 (l / 32) .. +7.  Within each group of 16 lanes,
// lane j addresses k row 8 (group / 2) + j / 4 (+ 4 for the high half) at
// units 16 (group % 2) + 4 (j % 4) .. +3, and the transposing read hands lane
// i of the group the four k values of unit 16 (group % 2) + i.  The 16
// 8-byte reads of a group fall in 16 distinct bank pairs.
__device__ __forceinline__ bf16x8 bh_slot_frag(const bf16_t* slot) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef v4i16 __attribute__((address_space(3))) * lds_v4p;
  const int lane = threadIdx.x & 63, G = lane >> 4, j = lane & 15;
  const int u = 16 * (G & 1) + 4 * (j & 3);
  const int c = 8 * (G >> 1) + (j >> 2);
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(slot + 32 * c + u));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(slot + 32 * (c + 4) + u));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// One chunk's results for the tile's rows: wave w holds, for each 32-row
// block i, pk[i][2g], pk[i][2g+1] = units 32w + 8g + 4 (l / 32) .. +3 of row
// 32i + l % 32 as bf16 pairs.  Each block goes through a staging tile (32
// rows x 256 units), so that the workgroup writes every row's 512 bytes of
// the chunk as whole 16-byte pieces of contiguous rows; out points at unit 0
// of the chunk in the tile's first row.  Block b of the kernel's sequence of
// blocks (b0 + i here) uses tile b % 2: the barrier after the writes of block
// b also orders block b - 1's reads before block b + 1's writes.
template <int MB>
__device__ __forceinline__ void bh_write_chunk(bf16_t* out, int h, int m,
                                               const uint32_t (&pk)[MB][8], bf16_t* St, int b0) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 31, q4 = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    bf16_t* T = St + ((b0 + i) & 1) * 32 * BH_SLD;
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint2*>(T + fr * BH_SLD + 32 * w + 8 * g + q4) =
          uint2{pk[i][2 * g], pk[i][2 * g + 1]};
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + j * BH_THREADS, r = c >> 5, piece = c & 31;
      if (32 * i + r < m)
        *reinterpret_cast<u32x4*>(out + (int64_t)(32 * i + r) * h + 8 * piece) =
            *reinterpret_cast<const u32x4*>(T + r * BH_SLD + 8 * piece);
    }
  }
}

// The tile's routed rows into the LDS tile (zeros past m up to the tile's
// 32-row blocks) and out to out[p0 + r] (the rows in expert order, for the
// table gradients): row r is src[src_row[r]], times scale[r] when scale is
// given (rounded to bf16 as the forward's gate-scaled products are).
template <int MB>
__device__ __forceinline__ void bh_gather_rows(const bf16_t* src, const int* src_row,
                                               const float* scale, int p0, int m, bf16_t* Rs,
                                               bf16_t* out) {
  constexpr int CPR = BH_D / 8;
  constexpr int XCH = 32 * MB * CPR;
  constexpr int XPT = (XCH + BH_THREADS - 1) / BH_THREADS;
  const int tid = threadIdx.x;
  u32x4 v[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = tid + i * BH_THREADS, r = c / CPR, cc = (c % CPR) * 8;
    v[i] = (c < XCH && r < m)
               ? *reinterpret_cast<const u32x4*>(src + (int64_t)src_row[r] * BH_D + cc)
               : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = tid + i * BH_THREADS, r = c / CPR, cc = (c % CPR) * 8;
    if (c < XCH) {
      u32x4 o = v[i];
      if (scale && r < m) {
        const float sc = scale[r];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[j] = cvt_pk_bf16(__uint_as_float(o[j] << 16) * sc,
                             __uint_as_float(o[j] & 0xffff0000u) * sc);
      }
      *reinterpret_cast<u32x4*>(Rs + r * BH_XLD + cc) = o;
      if (r < m) *reinterpret_cast<u32x4*>(out + (int64_t)(p0 + r) * BH_D + cc) = o;
    }
  }
}

// One tile of m <= 32 MB rows of expert e at positions p0 .. p0 + m - 1.
// The wave's table stream has 2 NA entries: NA = nch * BH_KS W1 fragments
// (chunk hc, k-step n: units hc*BH_H + 32w + lane%32, k = 16n + 8(lane/32)
// .. +7), then NA W2 pieces (chunk hc, k-step n: W2 row 16n + lane/4, units
// hc*BH_H + 32w + 8(lane%4) .. +7).  Entries past the end re-read the last
// one (a cache hit), so that every take issues a load and the ring keeps its
// depth across chunks and phases.
template <int MB, bool PACKED>
__device__ __forceinline__ void bh_tile(const BwHidFusedArgs& a, int e, int p0, int m,
                                        bf16_t* Rs, bf16_t* Ws, uint64_t* Mk, bf16_t* St,
                                        int* s_row, float* s_gate) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 31, fk = (lane >> 5) * 8, q4 = (lane >> 5) * 4;
  const int h = a.h, nch = h / BH_H, NA = nch * BH_KS, NS = 2 * NA;
  const bf16_t* w1e = (const bf16_t*)a.w1 + (int64_t)e * h * BH_D;
  const bf16_t* w2e = (const bf16_t*)a.w2 + (int64_t)e * BH_D * h;
  const bf16_t* wpe = (const bf16_t*)a.wp + (int64_t)e * nch * BH_WAVES * BH_PACK_NE * 512;
  auto frag = [&](int s) -> u32x4 {
    s = min(s, NS - 1);
    if (s < NA) {
      const int hc = s / BH_KS, n = s % BH_KS;
      if constexpr (PACKED)
        return *reinterpret_cast<const u32x4*>(
            wpe + (((int64_t)hc * BH_WAVES + w) * BH_PACK_NE + n) * 512 + lane * 8);
      else
        return *reinterpret_cast<const u32x4*>(w1e + (int64_t)(hc * BH_H + 32 * w + fr) * BH_D +
                                               16 * n + fk);
    }
    const int s2 = s - NA, hc = s2 / BH_KS, n = s2 % BH_KS;
    return *reinterpret_cast<const u32x4*>(w2e + (int64_t)(16 * n + (lane >> 2)) * h +
                                           hc * BH_H + 32 * w + 8 * (lane & 3));
  };
  u32x4 ring[BH_RING];
#pragma unroll
  for (int i = 0; i < BH_RING; ++i) ring[i] = frag(i);
  // entry s of the stream, held in ring slot i = s % BH_RING (passed as a
  // compile-time constant, so that the ring stays in registers)
  auto take = [&](int s, int i) -> u32x4 {
    const u32x4 v = ring[i];
    ring[i] = frag(s + BH_RING);
    return v;
  };

  // the routed rows' sources (token perm[p] / k) and gates
  if (tid < m) {
    const int asg = a.perm[p0 + tid];
    s_row[tid] = asg / a.k;
    s_gate[tid] = a.gate[asg];
  }
  __syncthreads();
  bh_gather_rows<MB>((const bf16_t*)a.x, s_row, nullptr, p0, m, Rs, (bf16_t*)a.xs);
  __syncthreads();
  bf16_t* hid = (bf16_t*)a.hid;
  bf16_t* dp = (bf16_t*)a.dp;

  // ---- phase A: a^T[units][rows] = W1[units] X^T; Hid = relu(a), signs ----
  for (int hc = 0; hc < nch; ++hc) {
    f32x16 sa[MB];
    bf16x8 xa[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      sa[i] = f32x16{};
      xa[i] = *reinterpret_cast<const bf16x8*>(Rs + (32 * i + fr) * BH_XLD + fk);
    }
#pragma unroll
    for (int ks = 0; ks < BH_KS; ++ks) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, take(hc * BH_KS + ks, ks % BH_RING));
      bf16x8 av[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i) av[i] = xa[i];
      if (ks + 1 < BH_KS) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
          xa[i] = *reinterpret_cast<const bf16x8*>(Rs + (32 * i + fr) * BH_XLD + (ks + 1) * 16 + fk);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) sa[i] = mfma32(b, av[i], sa[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // register group g of sa[i]: units 8g + q4 .. +3 of row 32i + fr
    uint64_t bits = 0;
    uint32_t pk[MB][8];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          bits |= (uint64_t)(sa[i][4 * g + j] > 0.f) << (16 * i + 4 * g + j);
        pk[i][2 * g] = cvt_pk_bf16(fmaxf(sa[i][4 * g], 0.f), fmaxf(sa[i][4 * g + 1], 0.f));
        pk[i][2 * g + 1] = cvt_pk_bf16(fmaxf(sa[i][4 * g + 2], 0.f), fmaxf(sa[i][4 * g + 3], 0.f));
      }
    }
    Mk[(hc * BH_WAVES + w) * 64 + lane] = bits;
    bh_write_chunk<MB>(hid + (int64_t)p0 * h + hc * BH_H, h, m, pk, St, hc * MB);
  }

  // ---- phase B: (dY W2)^T[units][rows] = W2^T[units] dY^T; dP ----
  __syncthreads();  // every wave is done with the x rows
  bh_gather_rows<MB>((const bf16_t*)a.dy, s_row, s_gate, p0, m, Rs, (bf16_t*)a.dys);
  __syncthreads();
  // the wave's LDS slot of 16 x 32 W2 elements: each piece is written after
  // the previous one has been read (one wave's LDS accesses complete in order)
  bf16_t* slot = Ws + w * 512;
  *reinterpret_cast<u32x4*>(slot + lane * 8) = take(NA, 0);
  bf16x8 wa = bh_slot_frag(slot);
  for (int hc = 0; hc < nch; ++hc) {
    f32x16 sd[MB];
    bf16x8 ya[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      sd[i] = f32x16{};
      ya[i] = *reinterpret_cast<const bf16x8*>(Rs + (32 * i + fr) * BH_XLD + fk);
    }
#pragma unroll
    for (int ks = 0; ks < BH_KS; ++ks) {
      // the next piece (of this chunk, the next one, or past the end) goes
      // through the slot and comes back as the next operand while this
      // k-step's MFMAs run
      *reinterpret_cast<u32x4*>(slot + lane * 8) = take(NA + hc * BH_KS + ks + 1, (ks + 1) % BH_RING);
      const bf16x8 wcur = wa;
      wa = bh_slot_frag(slot);
      bf16x8 av[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i) av[i] = ya[i];
      if (ks + 1 < BH_KS) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
          ya[i] = *reinterpret_cast<const bf16x8*>(Rs + (32 * i + fr) * BH_XLD + (ks + 1) * 16 + fk);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) sd[i] = mfma32(wcur, av[i], sd[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
    const uint64_t bits = Mk[(hc * BH_WAVES + w) * 64 + lane];
    uint32_t pk[MB][8];
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v[j] = ((bits >> (16 * i + 4 * g + j)) & 1u) ? sd[i][4 * g + j] : 0.f;
        pk[i][2 * g] = cvt_pk_bf16(v[0], v[1]);
        pk[i][2 * g + 1] = cvt_pk_bf16(v[2], v[3]);
      }
    }
    bh_write_chunk<MB>(dp + (int64_t)p0 * h + hc * BH_H, h, m, pk, St, (nch + hc) * MB);
  }
}

// This workgroup's tile, found from the routing offsets with the forward's
// fused-kernel numbering: expert e holds ceil(m_e / BH_M) tiles (m_e its
// rows), numbered in expert order, its 32-row blocks split over them by
// tile_rows.  Workgroup b takes tile (b % 8) * ceil(Q / 8) + b / 8 of the Q
// tiles, so that the tiles of an expert run on one XCD (workgroups go to the
// XCDs round-robin).  False for the workgroups past the last tile.  Every
// thread of the workgroup calls it (a block scan and two barriers).
__device__ __forceinline__ bool bh_find_tile(const int32_t* offsets, int E, int* e, int* p0,
                                             int* m) {
  __shared__ int s_info[3];
  const int tid = threadIdx.x;
  const int per = (E + BH_THREADS - 1) / BH_THREADS;  // experts per thread
  const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
  int nt = 0;
  for (int x = e0; x < e1; ++x) nt += (offsets[x + 1] - offsets[x] + BH_M - 1) / BH_M;
  int Q;
  int run = block_excl_scan<BH_THREADS>(nt, &Q);
  const int perx = (Q + 7) / 8;
  const int slot = blockIdx.x >> 3, q = (blockIdx.x & 7) * perx + slot;
  if (tid == 0) s_info[0] = -1;
  __syncthreads();
  if (slot < perx && q < Q && q >= run && q < run + nt) {
    for (int x = e0; x < e1; ++x) {
      const int o = offsets[x], mx = offsets[x + 1] - o, n = (mx + BH_M - 1) / BH_M;
      if (q < run + n) {
        int first, rows;
        tile_rows(mx, n, q - run, &first, &rows);
        s_info[0] = x;
        s_info[1] = o + first;
        s_info[2] = rows;
        break;
      }
      run += n;
    }
  }
  __syncthreads();
  *e = __builtin_amdgcn_readfirstlane(s_info[0]);
  *p0 = __builtin_amdgcn_readfirstlane(s_info[1]);
  *m = __builtin_amdgcn_readfirstlane(s_info[2]);
  return *e >= 0;
}

template <bool PACKED>
__global__ __launch_bounds__(BH_THREADS, 1) void bw_hidden_fused_kernel(BwHidFusedArgs a) {
  extern __shared__ __attribute__((aligned(16))) bf16_t bh_lds[];
  bf16_t* Rs = bh_lds;
  bf16_t* Ws = bh_lds + BH_M * BH_XLD;
  uint64_t* Mk = reinterpret_cast<uint64_t*>(Ws + BH_WAVES * 512);
  bf16_t* St = reinterpret_cast<bf16_t*>(Mk + BH_MAXCH * BH_WAVES * 64);
  __shared__ int s_row[BH_M];
  __shared__ float s_gate[BH_M];
  int e, p0, m;
  if (!bh_find_tile(a.offsets, a.E, &e, &p0, &m)) return;
  // only the 32-row blocks that hold rows run through the MFMAs
  const int mb = (m + 31) / 32;
  if (mb >= 3)
    bh_tile<3, PACKED>(a, e, p0, m, Rs, Ws, Mk, St, s_row, s_gate);
  else if (mb == 2)
    bh_tile<2, PACKED>(a, e, p0, m, Rs, Ws, Mk, St, s_row, s_gate);
  else
    bh_tile<1, PACKED>(a, e, p0, m, Rs, Ws, Mk, St, s_row, s_gate);
}

template <bool PACKED>
static hipError_t launch_bh(const BwHidFusedArgs& a, int64_t grid, hipStream_t s) {
  static bool attr_done = false;
  const size_t lds = bw_hidden_fused_lds();
  if (!attr_done) {
    hipError_t err = hipFuncSetAttribute((const void*)bw_hidden_fused_kernel<PACKED>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_done = true;
  }
  hipLaunchKernelGGL(bw_hidden_fused_kernel<PACKED>, dim3((unsigned)grid), dim3(BH_THREADS), lds,
                     s, a);
  return hipGetLastError();
}

hipError_t launch_bw_hidden_fused(const BwHidFusedArgs& a, int64_t A, hipStream_t s) {
  if (A == 0) return hipSuccess;
  const int64_t grid = bw_hidden_fused_grid(A, a.E);
  return a.wp ? launch_bh<true>(a, grid, s) : launch_bh<false>(a, grid, s);
}

// ---------------------------------------------------------------------------
// dX = dP W1 for the routed rows of the same tiles: dxs[p][c] = sum_u
// dp[p][u] W1[e][u][c], c < 512.  W1's contraction index (u) is its slow one,
// so its 16-unit by 32-column pieces take the per-wave LDS slot and the
// transposing read as W2 does in the hidden-layer kernel.  Wave w owns
// output columns 64w .. +63 (two 32-column blocks), the accumulators of the
// tile's rows stay in registers across the hidden chunks, and the tile's dP
// rows pass through LDS one chunk of 256 units at a time (two buffers: chunk
// hc + 1 is loaded into registers while chunk hc's MFMAs run).  The output
// leaves through LDS as 16-byte pieces of whole rows.
// ---------------------------------------------------------------------------
constexpr int BD_KS = BH_H / 16;   // k-steps per chunk (16 units each)

size_t bw_dx_fused_lds() {
  return sizeof(bf16_t) * (2 * (size_t)BH_M * BH_SLD + (size_t)BH_WAVES * 2 * 512);
}

template <int MB>
__device__ __forceinline__ void bd_tile(const BwDxFusedArgs& a, int e, int p0, int m, bf16_t* Ps,
                                        bf16_t* Ws) {
  constexpr int CPT = 2 * MB;  // 16-byte pieces of a dP chunk per thread
  static_assert((2 * BD_KS) % BH_RING == 0, "every chunk starts at ring slot 0");
  static_assert(2 * BH_M * BH_SLD >= BH_M * BH_XLD, "the output tile fits the dP buffers");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int fr = lane & 31, fk = (lane >> 5) * 8, q4 = (lane >> 5) * 4;
  const int h = a.h, nch = h / BH_H, NS = nch * BD_KS * 2;
  const bf16_t* w1e = (const bf16_t*)a.w1 + (int64_t)e * h * BH_D;
  const bf16_t* dp = (const bf16_t*)a.dp;
  // piece s: k-step s / 2 (units 16 (s / 2) .. +15: W1 row 16 (s / 2) + lane
  // / 4), column block s % 2 (columns 64w + 32 (s % 2) + 8 (lane % 4) .. +7)
  auto frag = [&](int s) -> u32x4 {
    s = min(s, NS - 1);
    return *reinterpret_cast<const u32x4*>(w1e + (int64_t)(16 * (s >> 1) + (lane >> 2)) * BH_D +
                                           64 * w + 32 * (s & 1) + 8 * (lane & 3));
  };
  u32x4 ring[BH_RING];
#pragma unroll
  for (int i = 0; i < BH_RING; ++i) ring[i] = frag(i);
  auto take = [&](int s, int i) -> u32x4 {
    const u32x4 v = ring[i];
    ring[i] = frag(s + BH_RING);
    return v;
  };
  // chunk hc of the tile's dP rows: piece c = tid + BH_THREADS i is row c /
  // 32, units hc * BH_H + 8 (c % 32) .. +7 (zeros past m)
  auto load_chunk = [&](int hc, u32x4 (&v)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * BH_THREADS, r = c >> 5;
      v[i] = r < m ? *reinterpret_cast<const u32x4*>(dp + (int64_t)(p0 + r) * h + hc * BH_H +
                                                     8 * (c & 31))
                   : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto put_chunk = [&](bf16_t* P, const u32x4 (&v)[CPT]) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + i * BH_THREADS;
      *reinterpret_cast<u32x4*>(P + (c >> 5) * BH_SLD + 8 * (c & 31)) = v[i];
    }
  };
  {
    u32x4 v[CPT];
    load_chunk(0, v);
    put_chunk(Ps, v);
  }
  // the wave's two LDS slots (one per column block) and the first k-step's
  // operands; each piece is written after the previous one in its slot has
  // been read (one wave's LDS accesses complete in order)
  bf16_t* sl0 = Ws + w * 1024;
  bf16_t* sl1 = sl0 + 512;
  *reinterpret_cast<u32x4*>(sl0 + lane * 8) = take(0, 0);
  *reinterpret_cast<u32x4*>(sl1 + lane * 8) = take(1, 1);
  bf16x8 wa0 = bh_slot_frag(sl0), wa1 = bh_slot_frag(sl1);
  f32x16 acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i][0] = acc[i][1] = f32x16{};
  __syncthreads();
  for (int hc = 0; hc < nch; ++hc) {
    const bf16_t* P = Ps + (hc & 1) * BH_M * BH_SLD;
    const bool more = hc + 1 < nch;
    u32x4 nv[CPT];
    if (more) load_chunk(hc + 1, nv);
    bf16x8 pa[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
      pa[i] = *reinterpret_cast<const bf16x8*>(P + (32 * i + fr) * BH_SLD + fk);
#pragma unroll
    for (int ks = 0; ks < BD_KS; ++ks) {
      // the next k-step's two pieces (this chunk's, the next one's first, or
      // past the end) go through the slots while this k-step's MFMAs run
      const int sn = 2 * (hc * BD_KS + ks + 1);
      *reinterpret_cast<u32x4*>(sl0 + lane * 8) = take(sn, (2 * ks + 2) % BH_RING);
      *reinterpret_cast<u32x4*>(sl1 + lane * 8) = take(sn + 1, (2 * ks + 3) % BH_RING);
      const bf16x8 c0 = wa0, c1 = wa1;
      wa0 = bh_slot_frag(sl0);
      wa1 = bh_slot_frag(sl1);
      bf16x8 av[MB];
#pragma unroll
      for (int i = 0; i < MB; ++i) av[i] = pa[i];
      if (ks + 1 < BD_KS) {
#pragma unroll
        for (int i = 0; i < MB; ++i)
          pa[i] = *reinterpret_cast<const bf16x8*>(P + (32 * i + fr) * BH_SLD + (ks + 1) * 16 + fk);
      }
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        acc[i][0] = mfma32(c0, av[i], acc[i][0]);
        acc[i][1] = mfma32(c1, av[i], acc[i][1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // the other buffer was last read in chunk hc - 1, before the previous barrier
    if (more) put_chunk(Ps + ((hc + 1) & 1) * BH_M * BH_SLD, nv);
    __syncthreads();
  }
  // dX -> bf16 -> LDS (the dP buffers) -> 16-byte pieces of whole rows;
  // register group g of acc[i][j] holds columns 64w + 32j + 8g + q4 .. +3 of
  // row 32i + fr
  bf16_t* O = Ps;
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<uint2*>(O + (32 * i + fr) * BH_XLD + 64 * w + 32 * j + 8 * g + q4) =
            uint2{cvt_pk_bf16(acc[i][j][4 * g], acc[i][j][4 * g + 1]),
                  cvt_pk_bf16(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3])};
  __syncthreads();
  bf16_t* dxs = (bf16_t*)a.dxs;
  for (int c = tid; c < m * (BH_D / 8); c += BH_THREADS) {
    const int r = c / (BH_D / 8), cc = (c % (BH_D / 8)) * 8;
    *reinterpret_cast<u32x4*>(dxs + (int64_t)(p0 + r) * BH_D + cc) =
        *reinterpret_cast<const u32x4*>(O + r * BH_XLD + cc);
  }
}

__global__ __launch_bounds__(BH_THREADS, 1) void bw_dx_fused_kernel(BwDxFusedArgs a) {
  extern __shared__ __attribute__((aligned(16))) bf16_t bd_lds[];
  bf16_t* Ps = bd_lds;
  bf16_t* Ws = bd_lds + 2 * BH_M * BH_SLD;
  int e, p0, m;
  if (!bh_find_tile(a.offsets, a.E, &e, &p0, &m)) return;
  const int mb = (m + 31) / 32;
  if (mb >= 3)
    bd_tile<3>(a, e, p0, m, Ps, Ws);
  else if (mb == 2)
    bd_tile<2>(a, e, p0, m, Ps, Ws);
  else
    bd_tile<1>(a, e, p0, m, Ps, Ws);
}

hipError_t launch_bw_dx_fused(const BwDxFusedArgs& a, int64_t A, hipStream_t s) {
  if (A == 0) return hipSuccess;
  static bool attr_done = false;
  const size_t lds = bw_dx_fused_lds();
  if (!attr_done) {
    hipError_t err = hipFuncSetAttribute((const void*)bw_dx_fused_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    attr_done = true;
  }
  hipLaunchKernelGGL(bw_dx_fused_kernel, dim3((unsigned)bw_hidden_fused_grid(A, a.E)),
                     dim3(BH_THREADS), lds, s, a);
  return hipGetLastError();
}

}  // namespace moe
