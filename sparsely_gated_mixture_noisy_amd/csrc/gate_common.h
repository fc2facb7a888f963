// Shared device code of the gate kernels, forward and backward: the tile
// geometry, the projection of a tile's rows onto a block of score tables on
// MFMA (bf16) or FMA (fp32), the noisy score, and DPP row reductions.  The
// backward kernels recompute the scores with this very code, so they see the
// forward's values bit for bit.
//
// Method ("MoE:稀疏门控混合专家", nengyongai.cn, sections 三 and 四):
//   clean_e = x . W_g[e] (+ bias_e),  H_e = clean_e + eps_e * softplus(x . W_noise[e]).
#pragma once
#include "moe_device.h"

namespace moe {

constexpr int GATE_ROWS = 32;
constexpr int GATE_WAVES = 8;
constexpr int GATE_THREADS = 64 * GATE_WAVES;
constexpr int GATE_BLOCK_E = 32 * GATE_WAVES;      // experts per projection block
constexpr int GATE_XLDS_MAX_D = 1024;               // input tile in LDS up to this d_model
constexpr int GATE_RING = 16;                       // table k-steps in flight per wave
constexpr int HLD = GATE_BLOCK_E + 1;               // LDS row stride of the score block

// A tile of RB blocks of 32 rows.
template <int RB>
struct GateTile {
  static constexpr int R = GATE_ROWS * RB;           // rows
  static constexpr int TPR = GATE_THREADS / R;       // selection lanes per row (16 or 8)
  static constexpr int NQ = GATE_BLOCK_E / TPR;      // scores per lane per expert block
  static_assert(TPR == 16 || TPR == 8, "a row's selection lanes lie inside one DPP row");
};

// Tile row held in accumulator register i of lane l (32x32 MFMA layout).
__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// Where a tile's input rows come from: global memory (rows[] tokens) or, for
// bf16 with d <= GATE_XLDS_MAX_D, an LDS copy Xs of the 32 rows.
template <typename T>
struct TileX {
  const T* x;
  const int* rows;
  const bf16_t* Xs;  // null: read x directly
  int xld;
};

// Where a block's table rows come from.  Unpacked: expert e is row row0 + e
// of wg / wn ([*][d]).  Packed (bf16, see launch_pack_gate): 32-expert block
// b of the group starts at block pk_blk0 + b of pk; per 64 columns it holds
// pk_nt tables x four 1 KB pieces, piece j of a table giving lane l the 16
// bytes the unpacked read of step j would give it.
struct GateTabs {
  const void* wg;
  const void* wn;
  int row0;
  const bf16_t* pk;
  int pk_blk0;
  int pk_nt;
};

// Copy the nr input rows of a tile to LDS (bf16, d % 8 == 0).
__device__ __forceinline__ void load_x_tile(const bf16_t* x, int d, const int* rows, int nr,
                                            bf16_t* Xs, int xld) {
  const int cpr = d / 8;
  for (int c = threadIdx.x; c < nr * cpr; c += GATE_THREADS) {
    const int r = c / cpr, cc = (c % cpr) * 8;
    *reinterpret_cast<u32x4*>(Xs + r * xld + cc) =
        *reinterpret_cast<const u32x4*>(x + (int64_t)rows[r] * d + cc);
  }
}

// Projection of one expert block: ac[i] = x[row] . wg[tab_row0 + e] and (NOISY)
// ar[i] = x[row] . wn[tab_row0 + e] for row = acc_row(i, lane) and
// e = blk + 32 * wave + (lane & 31).  Columns past E read a valid table row
// and are never used; waves with no valid column skip the MFMAs.  XLDS: the
// input rows are in the LDS tile Xs (bf16 only).
template <typename T, bool NOISY, bool XLDS, int RB = 1>
struct BlockProj;

// bf16: the contraction runs over groups of 64 columns.  Lane (c, h) of a
// wave (c = lane % 32, h = lane / 32) loads 64 contiguous bytes of its table
// row, columns 64G + 32h .. +31, as four 16-byte pieces j = 0..3; MFMA step j
// of the group pairs piece j (columns 64G + 32h + 8j .. +7) with the input
// columns at the same places.  The k order inside an MFMA is a permutation
// of the columns, the same for both operands, so every product term appears
// exactly once; the four loads of a piece run over whole cache lines back to
// back.  A ring of GATE_RING / 4 groups per table stays in flight.
template <bool NOISY, bool XLDS, int RB>
struct BlockProj<bf16_t, NOISY, XLDS, RB> {
  static constexpr int RG = RB == 1 ? GATE_RING / 4 : 2;  // groups in flight per table
  static __device__ __forceinline__ u32x4 ld(const bf16_t* p) {
    return *reinterpret_cast<const u32x4*>(p);
  }
  static __device__ __forceinline__ void run(const TileX<bf16_t>& tx, int d, const GateTabs& tb,
                                             int blk, int E, f32x16 (&ac)[RB],
                                             f32x16 (&ar)[RB]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane & 31, kh = (lane >> 5) * 32;
#pragma unroll
    for (int i = 0; i < RB; ++i) {
      ac[i] = f32x16{};
      ar[i] = f32x16{};
    }
    if (blk + w * 32 >= E) return;
    const int NG = d / 64;
    // table piece j of column group G sits at pg + G * gs + j * js
    const bf16_t *pg, *pn;
    int gs, js;
    if (tb.pk) {
      const int64_t b = tb.pk_blk0 + (blk >> 5) + w;
      pg = tb.pk + b * NG * tb.pk_nt * 2048 + lane * 8;
      pn = pg + 2048;
      gs = tb.pk_nt * 2048;
      js = 512;
    } else {
      const int64_t trow = tb.row0 + min(blk + w * 32 + c, E - 1);
      pg = (const bf16_t*)tb.wg + trow * d + kh;
      pn = NOISY ? (const bf16_t*)tb.wn + trow * d + kh : pg;
      gs = 64;
      js = 8;
    }
    const bf16_t* pa[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i)
      pa[i] = XLDS ? tx.Xs + (32 * i + c) * tx.xld + kh
                   : tx.x + (int64_t)tx.rows[32 * i + c] * d + kh;
    u32x4 rg[RG][4], rn[RG][4];
#pragma unroll
    for (int sl = 0; sl < RG; ++sl) {
      const int G = min(sl, NG - 1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        rg[sl][j] = ld(pg + G * gs + j * js);
        if (NOISY) rn[sl][j] = ld(pn + G * gs + j * js);
      }
    }
    int g = 0;
    for (; g + RG < NG; g += RG) {
#pragma unroll
      for (int sl = 0; sl < RG; ++sl) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int i = 0; i < RB; ++i) {
            const bf16x8 a = __builtin_bit_cast(bf16x8, ld(pa[i] + (g + sl) * 64 + j * 8));
            ac[i] = mfma32(a, __builtin_bit_cast(bf16x8, rg[sl][j]), ac[i]);
            if (NOISY) ar[i] = mfma32(a, __builtin_bit_cast(bf16x8, rn[sl][j]), ar[i]);
          }
        }
        // refill the slot with the group RG further on (the last one again
        // past the end)
        const int nx = min(g + RG + sl, NG - 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          rg[sl][j] = ld(pg + nx * gs + j * js);
          if (NOISY) rn[sl][j] = ld(pn + nx * gs + j * js);
        }
        // keep the refill ahead of the next slot's MFMAs
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // last groups: slots past NG carry duplicates and meet a zero input
#pragma unroll
    for (int sl = 0; sl < RG; ++sl) {
      const int G = min(g + sl, NG - 1);
      const bool live = g + sl < NG;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
          u32x4 av = ld(pa[i] + G * 64 + j * 8);
          if (!live) av = u32x4{0u, 0u, 0u, 0u};
          const bf16x8 a = __builtin_bit_cast(bf16x8, av);
          ac[i] = mfma32(a, __builtin_bit_cast(bf16x8, rg[sl][j]), ac[i]);
          if (NOISY) ar[i] = mfma32(a, __builtin_bit_cast(bf16x8, rn[sl][j]), ar[i]);
        }
      }
    }
  }
};

// fp32: plain FMA dot products, summed in k order.  The k loop runs outside
// the 16 rows (16 independent chains) and, when d % 4 == 0, four at a time on
// 16-byte loads.
template <bool NOISY, bool XLDS>
struct BlockProj<float, NOISY, XLDS, 1> {
  static __device__ __forceinline__ void run(const TileX<float>& tx, int d, const GateTabs& tb,
                                             int blk, int E, f32x16 (&acs)[1],
                                             f32x16 (&ars)[1]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    f32x16& ac = acs[0];
    f32x16& ar = ars[0];
    ac = f32x16{};
    ar = f32x16{};
    if (blk + w * 32 >= E) return;
    const int64_t trow = tb.row0 + min(blk + w * 32 + (lane & 31), E - 1);
    const float* pg = (const float*)tb.wg + trow * d;
    const float* pn = NOISY ? (const float*)tb.wn + trow * d : pg;
    const float* xr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) xr[i] = tx.x + (int64_t)tx.rows[acc_row(i, lane)] * d;
    int k = 0;
    if ((d & 3) == 0) {
      for (; k < d; k += 4) {
        const float4 g = *reinterpret_cast<const float4*>(pg + k);
        float4 n = g;
        if (NOISY) n = *reinterpret_cast<const float4*>(pn + k);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float4 xv = *reinterpret_cast<const float4*>(xr[i] + k);
          float c = ac[i];
          c = fmaf(xv.x, g.x, c);
          c = fmaf(xv.y, g.y, c);
          c = fmaf(xv.z, g.z, c);
          c = fmaf(xv.w, g.w, c);
          ac[i] = c;
          if (NOISY) {
            float r = ar[i];
            r = fmaf(xv.x, n.x, r);
            r = fmaf(xv.y, n.y, r);
            r = fmaf(xv.z, n.z, r);
            r = fmaf(xv.w, n.w, r);
            ar[i] = r;
          }
        }
      }
    }
    for (; k < d; ++k) {
      const float g = pg[k];
      const float n = NOISY ? pn[k] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float xv = xr[i][k];
        ac[i] = fmaf(xv, g, ac[i]);
        if (NOISY) ar[i] = fmaf(xv, n, ar[i]);
      }
    }
  }
};

// Cross-lane steps inside a 16-lane DPP row: the value of a partner lane.
// XOR1 / XOR2 swap neighbours and pairs (quad permutations); HALF_MIRROR
// pairs lane i with 7 - i of its half-row, MIRROR lane i with 15 - i.  Four
// steps in this order combine all 16 lanes of a row with any commutative,
// associative and idempotent operation (max, best-of).
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
// max over the TPR (16 or 8) lanes of a row (8 lanes: a half DPP row, which
// the first three steps cover)
template <int TPR>
__device__ __forceinline__ float row_max(float m) {
  m = fmaxf(m, dpp_f<DPP_XOR1>(m));
  m = fmaxf(m, dpp_f<DPP_XOR2>(m));
  m = fmaxf(m, dpp_f<DPP_HALF_MIRROR>(m));
  if constexpr (TPR == 16) m = fmaxf(m, dpp_f<DPP_MIRROR>(m));
  return m;
}
template <int CTRL>
__device__ __forceinline__ void best_step(float& bv, int& be) {
  const float v2 = dpp_f<CTRL>(bv);
  const int e2 = dpp_i<CTRL>(be);
  if (ranks_before(v2, e2, bv, be)) {
    bv = v2;
    be = e2;
  }
}

// The noisy score H = clean + eps * sp, rounded once (one fused multiply-add),
// so that every kernel that forms it gets the same value.
__device__ __forceinline__ float noisy_score(float clean, float eps, float sp) {
  return __builtin_fmaf(eps, sp, clean);
}

// The score a selection ranks: a NaN score (from a NaN input) ranks as -inf,
// so that every row still keeps k real experts (lowest index first among
// equals) and no sentinel index leaves the gate.
__device__ __forceinline__ float select_score(float h) {
  return __builtin_isnan(h) ? -INFINITY : h;
}

}  // namespace moe
