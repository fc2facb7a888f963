// Backward pass of the MoE layer with the flat gate: the gradients of
//   L = sum(dy * y) + w_imp * CV^2(Importance) + w_load * CV^2(Load)
// with respect to x, the gate tables and bias, and the expert tables.
//
// Pages: the reading note ("Outrageously Large Neural Networks — MoE 怎样让模型
// “很大但不每次全算”", sections 问题是什么 and 方法怎么做) says the hard choice of
// experts has no gradient and that the learnable noise lets more experts
// receive one; the paper card (ai-papers.xuzou.cn, sections 瓶颈 and 方法适配)
// names activation recomputation for the backward pass and the importance and
// load losses.  The kept set and the experts ranked k-th and (k+1)-th are held
// fixed; gradients flow through the kept softmax, the noisy scores, the smooth
// load estimate and the experts.
//
// Steps (one stream, in this order):
//   cv2 grad   dImp = w_imp dCV^2/dImportance, dLoad = w_load dCV^2/dLoad
//   gate out   dg[t,s] = dy_t . y_sorted[inv[t,s]] + dImp[e]; softmax
//              backward over the kept scores -> dHk[t,s]
//   gate rank  per token: which experts are ranked k-th and (k+1)-th, and the
//              sums of the threshold gradients that flow to their scores
//   gate grad  per (token, expert): dclean, draw (noise pre-activation), and
//              per-32-token partial sums of dclean (the bias gradient)
//   products   dx_gate = dclean W_g + draw W_noise;  dW_g = dclean^T x,
//              dW_noise = draw^T x (split over tokens, then summed in order)
//   experts    recompute the hidden layer, dHid = dY W2, its mask or SwiGLU
//              factors; dX = dP W1 (+ dB W3); dW1 = dP^T X; dW2 = dY^T Hid
//   assemble   dx_t = dx_gate_t + sum_s dX[inv[t,s]]
//
// bf16 layers: products run on MFMA (v_mfma_f32_32x32x16_bf16) with fp32
// accumulation; operands that are fp32 (dclean, draw) or scaled (gate * dy)
// are rounded to bf16 as they enter a product, the hidden activation and its
// gradients are rounded to bf16 between products, outputs are rounded to the
// layer's dtype.  fp32 layers use plain fp32 FMA loops.  Every sum runs in a
// fixed order: the results are deterministic.
#include "gate_common.h"
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// CV^2 gradients: g_i = w * 2 / (n m^2) * (v_i - m - var / m), fp64
// reductions in a fixed order; 0 when the mean is 0 or v is absent.
// ---------------------------------------------------------------------------
__device__ void cv2_grad_block(const float* v, int E, float wgt, float* g) {
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int i = tid; i < E; i += 256) s += (double)v[i];
  const double mean = sum256_f64<256>(s) / E;
  double q = 0.0;
  for (int i = tid; i < E; i += 256) {
    const double dv = (double)v[i] - mean;
    q += dv * dv;
  }
  const double var = sum256_f64<256>(q) / E;
  for (int i = tid; i < E; i += 256) {
    double r = 0.0;
    if (mean != 0.0) r = 2.0 / ((double)E * mean * mean) * ((double)v[i] - mean - var / mean);
    g[i] = (float)((double)wgt * r);
  }
}

__global__ __launch_bounds__(256) void bw_cv2_grad_kernel(const float* imp, const float* load,
                                                          int E, float wi, float wl, float* dimp,
                                                          float* dload) {
  if (imp) {
    cv2_grad_block(imp, E, wi, dimp);
  } else {
    for (int i = threadIdx.x; i < E; i += 256) dimp[i] = 0.f;
  }
  if (load) {
    cv2_grad_block(load, E, wl, dload);
  } else {
    for (int i = threadIdx.x; i < E; i += 256) dload[i] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// Gate outputs: one wave per token.  dg[s] = dy_t . y_sorted[inv[t*k+s]]
// (lanes over d, then a fixed butterfly) + dImp[idx[t,s]]; then
// dHk[t,s] = g_s (dg_s - sum_j g_j dg_j).
// ---------------------------------------------------------------------------
// Four consecutive elements as floats (8-byte bf16 or 16-byte fp32 load).
template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]) {
  if constexpr (sizeof(T) == 2) {
    const uint2 x = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xffff0000u);
    v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xffff0000u);
  } else {
    const float4 x = *reinterpret_cast<const float4*>(p);
    v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
  }
}

// This lane's share of the dot product of two d-element rows (lanes over d;
// the caller reduces over the wave).
template <typename T>
__device__ __forceinline__ float row_dot(const T* u, const T* v, int d, int lane) {
  float acc = 0.f;
  if ((d & 3) == 0) {
    // four elements per lane and step: 8-byte (bf16) or 16-byte (fp32) loads
    for (int c = lane * 4; c < d; c += 256) {
      float a[4], b[4];
      if constexpr (sizeof(T) == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(u + c);
        const uint2 y = *reinterpret_cast<const uint2*>(v + c);
        a[0] = __uint_as_float(x.x << 16); a[1] = __uint_as_float(x.x & 0xffff0000u);
        a[2] = __uint_as_float(x.y << 16); a[3] = __uint_as_float(x.y & 0xffff0000u);
        b[0] = __uint_as_float(y.x << 16); b[1] = __uint_as_float(y.x & 0xffff0000u);
        b[2] = __uint_as_float(y.y << 16); b[3] = __uint_as_float(y.y & 0xffff0000u);
      } else {
        const float4 x = *reinterpret_cast<const float4*>(u + c);
        const float4 y = *reinterpret_cast<const float4*>(v + c);
        a[0] = x.x; a[1] = x.y; a[2] = x.z; a[3] = x.w;
        b[0] = y.x; b[1] = y.y; b[2] = y.z; b[3] = y.w;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = fmaf(a[j], b[j], acc);
    }
  } else {
    for (int c = lane; c < d; c += 64) acc = fmaf(Elem<T>::load(u, c), Elem<T>::load(v, c), acc);
  }
  return acc;
}

// dg[s] = dy_t . y_sorted[inv[t*k+s]] (+ dImp of the slot's expert) and the
// slot's gate, for the k slots of token t (k <= 8).  Each column chunk of dy
// is loaded once and the k slots' rows are loaded together, so their loads
// are in flight at the same time; every slot sums its products in column
// order, then reduces over the wave.
template <typename T>
__device__ __forceinline__ void slot_grads(const void* dyp, const void* ysp, const int32_t* inv,
                                           const int32_t* idx, const float* gate,
                                           const float* dimp, int64_t t, int k, int d, int lane,
                                           float (&dg)[8], float (&g)[8]) {
  const T* dy = (const T*)dyp + t * d;
  const T* ys = (const T*)ysp;
  int64_t p[8];
  float acc[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    // a slot dropped by a capacity (inv = -1) contributes nothing to y
    p[s] = s < k ? inv[t * k + s] : -1;
    g[s] = s < k ? gate[t * k + s] : 0.f;
    acc[s] = 0.f;
  }
  if ((d & 3) == 0) {
    // four elements per lane and step: 8-byte (bf16) or 16-byte (fp32) loads
    for (int c = lane * 4; c < d; c += 256) {
      float u[4], v[8][4];
      if constexpr (sizeof(T) == 2) {
        const uint2 x = *reinterpret_cast<const uint2*>(dy + c);
        u[0] = __uint_as_float(x.x << 16); u[1] = __uint_as_float(x.x & 0xffff0000u);
        u[2] = __uint_as_float(x.y << 16); u[3] = __uint_as_float(x.y & 0xffff0000u);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const uint2 y = p[s] >= 0 ? *reinterpret_cast<const uint2*>(ys + p[s] * d + c)
                                    : uint2{0u, 0u};
          v[s][0] = __uint_as_float(y.x << 16); v[s][1] = __uint_as_float(y.x & 0xffff0000u);
          v[s][2] = __uint_as_float(y.y << 16); v[s][3] = __uint_as_float(y.y & 0xffff0000u);
        }
      } else {
        const float4 x = *reinterpret_cast<const float4*>(dy + c);
        u[0] = x.x; u[1] = x.y; u[2] = x.z; u[3] = x.w;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float4 y = p[s] >= 0 ? *reinterpret_cast<const float4*>(ys + p[s] * d + c)
                                     : float4{0.f, 0.f, 0.f, 0.f};
          v[s][0] = y.x; v[s][1] = y.y; v[s][2] = y.z; v[s][3] = y.w;
        }
      }
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[s] = fmaf(u[j], v[s][j], acc[s]);
    }
  } else {
    for (int c = lane; c < d; c += 64) {
      const float u = Elem<T>::load(dy, c);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (p[s] >= 0) acc[s] = fmaf(u, Elem<T>::load(ys, p[s] * d + c), acc[s]);
    }
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    dg[s] = 0.f;
    if (s < k) {
      dg[s] = wave_sum(acc[s]);
      if (dimp) dg[s] += dimp[idx[t * k + s]];
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void bw_gate_out_kernel(BwGateOutArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  float dg[8], g[8];
  slot_grads<T>(a.dy, a.y_sorted, a.inv, a.idx, a.gate, a.dimp, t, a.k, a.d, lane, dg, g);
  float sdot = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) sdot = fmaf(g[s], dg[s], sdot);
  if (lane < a.k) {
    float v = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s == lane) v = g[s] * (dg[s] - sdot);
    a.dhk[t * a.k + lane] = v;
  }
}

// ---------------------------------------------------------------------------
// The hierarchy's gate, one wave per token.  The k slots are group-major: the
// kpg slots of kept group a are a*kpg .. a*kpg+kpg-1.  A kept gate is
// gp_a gs_s (primary weight of the group times secondary weight of the
// expert); gp_a is the sum of the group's gates and gs_s = gate_s / gp_a.
// With V_a = sum of gs dg over the group (the gradient of gp_a), the
// secondary score gradient is dHs_s = gate_s (dg_s - V_a) and the primary
// one dHp_a = gp_a (V_a - sum over kept groups of gp V).  Noisy scores H = clean + eps *
// softplus(raw) add d raw = dH * eps * sigmoid(raw).  dx's share is
// sum over slots of (dHs W_gate[e] + d raw W_noise[e]) plus the same over the
// kept groups with the primary tables, in that fixed order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bw_hier_gate_kernel(BwHierGateArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.T) return;
  const int k = a.k, kpg = a.kpg, d = a.d, Eg = a.Eg, G = a.G;
  const bool noisy = a.w_noise != nullptr;
  const bool noisy_p = a.w_noise_p != nullptr;
  float dg[8], g[8];
  slot_grads<T>(a.dy, a.y_sorted, a.inv, a.idx, a.gate, a.dimp, t, k, d, lane, dg, g);
  int e[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) e[s] = s < k ? a.idx[t * k + s] : 0;
  // per slot, of its group (groups are runs of kpg slots): gp = the group's
  // primary weight (sum of its product gates), gs = gate / gp its secondary
  // weight, V = sum of gs * dg over the group (the primary weight's gradient)
  float gpg[8], gs[8], V[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    float gp = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < k && u / kpg == s / kpg) gp += g[u];
    gpg[s] = gp;
    gs[s] = gp > 0.f ? g[s] / gp : 0.f;
  }
  float tot = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    float v = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < k && u / kpg == s / kpg) v = fmaf(gs[u], dg[u], v);
    V[s] = v;
    if (s < k && s % kpg == 0) tot += gpg[s];
  }
  // primary softmax weights renormalised (their sum is 1 up to rounding, so
  // a single kept group gets exactly 1 and no gradient)
  float PV = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s)
    if (s < k && s % kpg == 0) PV = fmaf(gpg[s] / tot, V[s], PV);
  const T* xr = (const T*)a.x + t * d;
  // the raw noise scores of the kept experts and groups: all rows' loads in
  // flight together, then one wave reduction each
  float rw[8], rp[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) rw[s] = rp[s] = 0.f;
  const T* wn = (const T*)a.w_noise;
  const T* wnp = (const T*)a.w_noise_p;
  if (noisy || noisy_p) {
    if ((d & 3) == 0) {
      for (int c = lane * 4; c < d; c += 256) {
        float xv[4];
        load4<T>(xr + c, xv);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          if (s >= k) continue;
          if (noisy) {
            float v[4];
            load4<T>(wn + (int64_t)e[s] * d + c, v);
#pragma unroll
            for (int j = 0; j < 4; ++j) rw[s] = fmaf(xv[j], v[j], rw[s]);
          }
          if (noisy_p && s % kpg == 0) {
            float v[4];
            load4<T>(wnp + (int64_t)(e[s] / Eg) * d + c, v);
#pragma unroll
            for (int j = 0; j < 4; ++j) rp[s] = fmaf(xv[j], v[j], rp[s]);
          }
        }
      }
    } else {
      for (int c = lane; c < d; c += 64) {
        const float xv = Elem<T>::load(xr, c);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          if (s >= k) continue;
          if (noisy) rw[s] = fmaf(xv, Elem<T>::load(wn, (int64_t)e[s] * d + c), rw[s]);
          if (noisy_p && s % kpg == 0)
            rp[s] = fmaf(xv, Elem<T>::load(wnp, (int64_t)(e[s] / Eg) * d + c), rp[s]);
        }
      }
    }
  }
  float cs[8], ns[8], cp[8], np_[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    cs[s] = ns[s] = cp[s] = np_[s] = 0.f;
    if (s >= k) continue;
    cs[s] = g[s] * (dg[s] - V[s]);
    const int grp = e[s] / Eg, j = e[s] % Eg;
    if (noisy) {
      const float raw = wave_sum(rw[s]);
      ns[s] = cs[s] * a.noise.at(t, grp, G, j, Eg) / (1.0f + __expf(-raw));
    }
    if (s % kpg == 0) {  // the group's first slot carries its primary gradients
      cp[s] = gpg[s] / tot * (V[s] - PV);
      if (noisy_p) {
        const float raw = wave_sum(rp[s]);
        np_[s] = cp[s] * a.noise_p.at(t, 0, 1, grp, G) / (1.0f + __expf(-raw));
      }
    }
  }
  if (lane < k) {
    float c = 0.f, n = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s == lane) {
        c = cs[s];
        n = ns[s];
      }
    a.cs[t * k + lane] = c;
    if (a.ns) a.ns[t * k + lane] = n;
  }
  for (int gg = lane; gg < G; gg += 64) {
    float c = 0.f, n = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < k && s % kpg == 0 && e[s] / Eg == gg) {
        c = cp[s];
        n = np_[s];
      }
    a.dcp[t * G + gg] = c;
    if (a.drp) a.drp[t * G + gg] = n;
  }
  const T* wg = (const T*)a.w_gate;
  const T* wgp = (const T*)a.w_gate_p;
  if ((d & 3) == 0) {
    // four columns per lane and step, every table row's chunk loaded together
    for (int c = lane * 4; c < d; c += 256) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s >= k) continue;
        float v[4], u[4];
        load4<T>(wg + (int64_t)e[s] * d + c, v);
        if (noisy) load4<T>(wn + (int64_t)e[s] * d + c, u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j] = fmaf(cs[s], v[j], acc[j]);
          if (noisy) acc[j] = fmaf(ns[s], u[j], acc[j]);
        }
      }
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        if (s >= k || s % kpg != 0) continue;
        const int64_t grp = e[s] / Eg;
        float v[4], u[4];
        load4<T>(wgp + grp * d + c, v);
        if (noisy_p) load4<T>(wnp + grp * d + c, u);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[j] = fmaf(cp[s], v[j], acc[j]);
          if (noisy_p) acc[j] = fmaf(np_[s], u[j], acc[j]);
        }
      }
      *reinterpret_cast<float4*>(a.dxg + t * d + c) = float4{acc[0], acc[1], acc[2], acc[3]};
    }
    return;
  }
  for (int c = lane; c < d; c += 64) {
    float acc = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s >= k) continue;
      acc = fmaf(cs[s], Elem<T>::load(wg, (int64_t)e[s] * d + c), acc);
      if (noisy) acc = fmaf(ns[s], Elem<T>::load(wn, (int64_t)e[s] * d + c), acc);
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s >= k || s % kpg != 0) continue;
      const int64_t grp = e[s] / Eg;
      acc = fmaf(cp[s], Elem<T>::load(wgp, grp * d + c), acc);
      if (noisy_p) acc = fmaf(np_[s], Elem<T>::load(wnp, grp * d + c), acc);
    }
    a.dxg[t * d + c] = acc;
  }
}

// ---------------------------------------------------------------------------
// Per-expert weighted row sums: out[e] = sum over the expert's rows, in
// routed order, of coefficient * x row.  One workgroup per (expert, 256
// columns); rows in batches of 8 so that their loads are in flight together.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void bw_expert_rowsum_kernel(BwRowSumArgs a) {
  const int e = blockIdx.x;
  const int c = blockIdx.y * 256 + threadIdx.x;
  if (c >= a.d) return;
  const int lo = a.offsets[e], hi = a.offsets[e + 1];
  const T* x = (const T*)a.x;
  float s0 = 0.f, s1 = 0.f;
  for (int p = lo; p < hi; p += 8) {
    int r[8];
    float v[8], c0[8], c1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) r[u] = p + u < hi ? a.perm[p + u] : -1;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      v[u] = r[u] >= 0 ? Elem<T>::load(x, (int64_t)(r[u] / a.k) * a.d + c) : 0.f;
      c0[u] = r[u] >= 0 ? a.c0[r[u]] : 0.f;
      c1[u] = r[u] >= 0 && a.c1 ? a.c1[r[u]] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (r[u] < 0) continue;
      s0 = fmaf(c0[u], v[u], s0);
      s1 = fmaf(c1[u], v[u], s1);
    }
  }
  Elem<T>::store((T*)a.out0, (int64_t)e * a.d + c, s0);
  if (a.out1) Elem<T>::store((T*)a.out1, (int64_t)e * a.d + c, s1);
}

// ---------------------------------------------------------------------------
// Gate score tiles (32 tokens, eight waves, experts in blocks of 256): the
// forward's projection recomputes clean = x W_g^T + b, raw = x W_noise^T and
// H for the lane's (row, expert) pairs in the MFMA accumulator layout (lane l
// of wave w: expert blk + 32w + l%32, rows acc_row(i, l)).
// ---------------------------------------------------------------------------
struct RankBest {
  float v;
  int e;
};
// a ranks before b: larger score, then lower index
__device__ __forceinline__ bool rb_before(const RankBest& a, const RankBest& b) {
  return ranks_before(a.v, a.e, b.v, b.e);
}

// The rank step's reductions over the 32 lanes of a half-wave (one row, 32
// experts) run on DPP moves: quad swaps, half-row and row mirrors, then the
// lower row's total broadcast into the upper row (lanes 16-31 and 48-63 end
// with the half-wave's result).  Each step combines two equal partial results,
// so the sums follow the balanced tree of an xor butterfly, bit for bit.
constexpr int DPP_BCAST15 = 0x142;
template <int CTRL, int ROWS>
__device__ __forceinline__ RankBest rb_dpp(const RankBest& r) {  // rows outside ROWS: r
  return RankBest{__builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                      __builtin_bit_cast(int, r.v), __builtin_bit_cast(int, r.v), CTRL, ROWS, 0xF,
                      false)),
                  __builtin_amdgcn_update_dpp(r.e, r.e, CTRL, ROWS, 0xF, false)};
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float sum_dpp(float v) {  // rows outside ROWS: 0
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ void rank_step(RankBest& wk, RankBest& bd, float& sk, float& sd) {
  const RankBest ok = rb_dpp<CTRL, ROWS>(wk);
  if (rb_before(wk, ok)) wk = ok;
  const RankBest od = rb_dpp<CTRL, ROWS>(bd);
  if (rb_before(od, bd)) bd = od;
  sk += sum_dpp<CTRL, ROWS>(sk);
  sd += sum_dpp<CTRL, ROWS>(sd);
}
// worst kept and best dropped expert, and the two sums, over the half-wave
__device__ __forceinline__ void rank_half_reduce(RankBest& wk, RankBest& bd, float& sk, float& sd) {
  rank_step<DPP_XOR1, 0xF>(wk, bd, sk, sd);
  rank_step<DPP_XOR2, 0xF>(wk, bd, sk, sd);
  rank_step<DPP_HALF_MIRROR, 0xF>(wk, bd, sk, sd);
  rank_step<DPP_MIRROR, 0xF>(wk, bd, sk, sd);
  rank_step<DPP_BCAST15, 0xA>(wk, bd, sk, sd);
}
constexpr int RANK_LANE = 31;  // the half-wave lane that holds the reductions

// The gate tile's shared set-up: rows, the x tile, kept masks (bit r of
// sb[e]: tile row r keeps expert e), kept experts per row, thresholds.
struct BwTileShared {
  int rows[GATE_ROWS];
  int kle[GATE_ROWS][8];
  float kth[GATE_ROWS], k1th[GATE_ROWS];
};

template <typename T, bool XLDS>
__device__ void bw_tile_setup(const BwGateArgs& a, BwTileShared& sh, uint32_t* sb, bf16_t* Xs,
                              int xld) {
  const int tid = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * GATE_ROWS;
  if (tid < GATE_ROWS) sh.rows[tid] = (int)min<int64_t>(t0 + tid, a.T - 1);
  for (int i = tid; i < a.E; i += GATE_THREADS) sb[i] = 0u;
  // the rows' kept experts and thresholds are requested before the x tile,
  // so that the tile's wait covers them too
  const int64_t t = t0 + tid;
  const bool valid = tid < GATE_ROWS && t < a.T;
  int ke[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) ke[s] = (valid && s < a.k) ? a.idx[t * a.k + s] : -1;
  const float kth = (valid && a.thr) ? a.thr[2 * t] : 0.f;
  const float k1th = (valid && a.thr) ? a.thr[2 * t + 1] : 0.f;
  __syncthreads();
  if (XLDS) load_x_tile((const bf16_t*)a.x, a.d, sh.rows, GATE_ROWS, Xs, xld);
  if (tid < GATE_ROWS) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      sh.kle[tid][s] = ke[s];
      if (ke[s] >= 0) atomicOr(&sb[ke[s]], 1u << tid);
    }
    sh.kth[tid] = kth;
    sh.k1th[tid] = k1th;
  }
  __syncthreads();
}

// Scores of one expert block for the lane: clean (bias included), sp, H, raw.
template <typename T, bool NOISY, bool XLDS>
__device__ __forceinline__ void bw_block_scores(const BwGateArgs& a, const BwTileShared& sh,
                                                const bf16_t* Xs, int xld, int blk, f32x16& cs,
                                                f32x16& ss, f32x16& hs, f32x16& rs, f32x16& es) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = blk + w * 32 + (lane & 31);
  const bool ev = e < a.E;
  if (NOISY) {
    float ev16[16];
    a.noise.rows16(0, 1, e, a.E, [&](int r) { return sh.rows[acc_row(r, lane)]; }, ev16);
#pragma unroll
    for (int r = 0; r < 16; ++r) es[r] = ev ? ev16[r] : 0.f;
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) es[r] = 0.f;
  }
  const TileX<T> tx{(const T*)a.x, sh.rows, XLDS ? Xs : nullptr, xld};
  const GateTabs tb{a.w_gate, a.w_noise, 0, (const bf16_t*)a.w_pack, 0, a.pack_nt};
  f32x16 ac[1], ar[1];
  BlockProj<T, NOISY, XLDS, 1>::run(tx, a.d, tb, blk, a.E, ac, ar);
  const float b = (a.bias && ev) ? a.bias[e] : 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const float c = ac[0][r] + b;
    cs[r] = c;
    if (NOISY) {
      const float sp = softplus_f(ar[0][r]);
      ss[r] = sp;
      hs[r] = select_score(noisy_score(c, es[r], sp));
      rs[r] = ar[0][r];
    } else {
      ss[r] = 0.f;
      hs[r] = select_score(c);
      rs[r] = 0.f;
    }
  }
}

// phi(z) = exp(-z^2/2) / sqrt(2 pi); z = +-inf gives 0
__device__ __forceinline__ float normal_pdf_f(float z) {
  return 0.3989422804014327f * exp2_hw(-0.5f * z * z * 1.4426950408889634f);
}

// Each expert block's candidates are reduced over the half-wave right away
// and merged into the wave's LDS slots, so no per-row state lives through the
// projections (carried through them, it made the kernel spill 300 bytes per
// lane).
template <typename T, bool NOISY, bool XLDS>
__global__ __launch_bounds__(GATE_THREADS) void bw_gate_rank_kernel(BwGateArgs a) {
  __shared__ BwTileShared sh;
  __shared__ RankBest wk[GATE_WAVES][GATE_ROWS], bn[GATE_WAVES][GATE_ROWS];
  __shared__ float wsk[GATE_WAVES][GATE_ROWS], wsn[GATE_WAVES][GATE_ROWS];
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int xld = a.d + 8;
  bf16_t* Xs = reinterpret_cast<bf16_t*>(dyn);
  uint32_t* sb = reinterpret_cast<uint32_t*>(dyn + (XLDS ? sizeof(bf16_t) * GATE_ROWS * xld : 0));
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid < GATE_WAVES * GATE_ROWS) {
    const int ww = tid / GATE_ROWS, row = tid % GATE_ROWS;
    wk[ww][row] = RankBest{INFINITY, -1};
    bn[ww][row] = RankBest{-INFINITY, 0x7fffffff};
    wsk[ww][row] = 0.f;
    wsn[ww][row] = 0.f;
  }
  bw_tile_setup<T, XLDS>(a, sh, sb, Xs, xld);
  __syncthreads();
  const bool smooth = NOISY && a.dload != nullptr;
  for (int blk = 0; blk < a.E; blk += GATE_BLOCK_E) {
    f32x16 cs, ss, hs, rs, es;
    bw_block_scores<T, NOISY, XLDS>(a, sh, Xs, xld, blk, cs, ss, hs, rs, es);
    RankBest worst_kept[16], best_drop[16];
    float s_kept[16], s_drop[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      worst_kept[r] = RankBest{INFINITY, -1};
      best_drop[r] = RankBest{-INFINITY, 0x7fffffff};
      s_kept[r] = 0.f;
      s_drop[r] = 0.f;
    }
    const int e = blk + w * 32 + (lane & 31);
    if (e < a.E) {
      const uint32_t km = sb[e];
      const float dl = smooth ? a.dload[e] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, lane);
        const bool kept = (km >> row) & 1u;
        const RankBest cur{hs[r], e};
        if (kept) {
          if (rb_before(worst_kept[r], cur)) worst_kept[r] = cur;
        } else {
          if (rb_before(cur, best_drop[r])) best_drop[r] = cur;
        }
        if (smooth) {
          const float th = kept ? sh.k1th[row] : sh.kth[row];
          const float isp = rcp_hw(ss[r]);
          const float z = (cs[r] - th) * isp;
          const float dt = (z == INFINITY || z == -INFINITY) ? 0.f : -dl * normal_pdf_f(z) * isp;
          if (kept) s_kept[r] += dt;
          else s_drop[r] += dt;
        }
      }
    }
    // across the 32 lanes of a half-wave (the experts of one row in this block)
#pragma unroll
    for (int r = 0; r < 16; ++r) rank_half_reduce(worst_kept[r], best_drop[r], s_kept[r], s_drop[r]);
    // into the wave's slots, block after block (each row's slot has one writer)
    if ((lane & 31) == RANK_LANE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, lane);
        if (rb_before(wk[w][row], worst_kept[r])) wk[w][row] = worst_kept[r];
        if (rb_before(best_drop[r], bn[w][row])) bn[w][row] = best_drop[r];
        wsk[w][row] += s_kept[r];
        wsn[w][row] += s_drop[r];
      }
    }
  }
  __syncthreads();
  // across the eight waves, in wave order
  if (tid < GATE_ROWS) {
    const int64_t t = (int64_t)blockIdx.x * GATE_ROWS + tid;
    RankBest k0 = wk[0][tid], d0 = bn[0][tid];
    float sk = wsk[0][tid], sd = wsn[0][tid];
    for (int i = 1; i < GATE_WAVES; ++i) {
      if (rb_before(k0, wk[i][tid])) k0 = wk[i][tid];
      if (rb_before(bn[i][tid], d0)) d0 = bn[i][tid];
      sk += wsk[i][tid];
      sd += wsn[i][tid];
    }
    if (t < a.T) {
      int4 out;
      out.x = k0.e;                                   // expert ranked k-th
      out.y = d0.e == 0x7fffffff ? -1 : d0.e;         // ranked k+1-th (none: -1)
      out.z = __float_as_int(sd);                     // gradient to the k-th score
      out.w = __float_as_int(sk);                     // gradient to the (k+1)-th score
      reinterpret_cast<int4*>(a.rinfo)[t] = out;
    }
  }
}

// v as bf16 hi = rne(v) and lo = rne(v - hi), the halves the products take
__device__ __forceinline__ void split_store(bf16_t* hi, bf16_t* lo, int64_t i, float v) {
  const uint32_t h = cvt_pk_bf16(v, 0.f) << 16;
  hi[i] = (bf16_t)(h >> 16);
  lo[i] = (bf16_t)(cvt_pk_bf16(v - __uint_as_float(h), 0.f) & 0xffffu);
}

// LDS row stride (bf16 elements) of the fused dx product's score-gradient tiles
constexpr int BWD_LD = GATE_BLOCK_E + 8;
constexpr size_t BWD_LDS = sizeof(bf16_t) * 4 * GATE_ROWS * BWD_LD;

// DXG (bf16, E <= GATE_BLOCK_E): also form the tile's dx_gate = dclean W_gate
// + draw W_noise on MFMA, from the score gradients staged in LDS as bf16
// hi + lo halves (the split the separate product uses) and the transposed
// tables: wave w takes the 32-column blocks w, w + 8, ...; an accumulator lane
// holds four consecutive columns of one row.
// RANK (E <= GATE_BLOCK_E, one expert block): the rank step runs here, on the
// scores this kernel holds anyway, with the rank kernel's operations in its
// order (one block: each wave's slot takes its half-wave's result as is), so
// the projections are computed once instead of twice.
__device__ __forceinline__ void rank_in_registers(const f32x16& cs, const f32x16& ss,
                                                  const f32x16& hs, int e, int E,
                                                  const uint32_t* sb, const BwTileShared& sh,
                                                  const float* dload, bool smooth,
                                                  RankBest (&wk)[GATE_WAVES][GATE_ROWS],
                                                  RankBest (&bn)[GATE_WAVES][GATE_ROWS],
                                                  float (&wsk)[GATE_WAVES][GATE_ROWS],
                                                  float (&wsn)[GATE_WAVES][GATE_ROWS],
                                                  int4* ri, int64_t t0, int64_t T) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const bool live = e < E;
  const uint32_t km = live ? sb[e] : 0u;
  const float dl = (smooth && live) ? dload[e] : 0.f;
  // one accumulator row at a time, reduced over the half-wave and parked in
  // LDS at once, so that nothing of it stays live across rows
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = acc_row(r, lane);
    RankBest worst_kept{INFINITY, -1}, best_drop{-INFINITY, 0x7fffffff};
    float s_kept = 0.f, s_drop = 0.f;
    if (live) {
      const bool kept = (km >> row) & 1u;
      const RankBest cur{hs[r], e};
      if (kept) worst_kept = cur;
      else best_drop = cur;
      if (smooth) {
        const float th = kept ? sh.k1th[row] : sh.kth[row];
        const float isp = rcp_hw(ss[r]);
        const float z = (cs[r] - th) * isp;
        const float dt = (z == INFINITY || z == -INFINITY) ? 0.f : -dl * normal_pdf_f(z) * isp;
        if (kept) s_kept += dt;
        else s_drop += dt;
      }
    }
    rank_half_reduce(worst_kept, best_drop, s_kept, s_drop);
    if ((lane & 31) == RANK_LANE) {
      wk[w][row] = worst_kept;
      bn[w][row] = best_drop;
      wsk[w][row] = 0.f + s_kept;
      wsn[w][row] = 0.f + s_drop;
    }
  }
  __syncthreads();
  if (tid < GATE_ROWS) {
    RankBest k0 = wk[0][tid], d0 = bn[0][tid];
    float sk = wsk[0][tid], sd = wsn[0][tid];
    for (int i = 1; i < GATE_WAVES; ++i) {
      if (rb_before(k0, wk[i][tid])) k0 = wk[i][tid];
      if (rb_before(bn[i][tid], d0)) d0 = bn[i][tid];
      sk += wsk[i][tid];
      sd += wsn[i][tid];
    }
    int4 out;
    out.x = k0.e;
    out.y = d0.e == 0x7fffffff ? -1 : d0.e;
    out.z = __float_as_int(sd);
    out.w = __float_as_int(sk);
    ri[tid] = out;
  }
  __syncthreads();
}

template <typename T, bool NOISY, bool XLDS, bool DXG, bool RANK = false>
__global__ __launch_bounds__(GATE_THREADS) void bw_gate_grad_kernel(BwGateArgs a) {
  __shared__ BwTileShared sh;
  __shared__ int4 ri[GATE_ROWS];
  __shared__ float dhk[GATE_ROWS][8];
  // the tile's gradients to H from the kept gates and the threshold terms, by
  // (row, expert of the block); zero elsewhere
  __shared__ float dhm[GATE_ROWS][GATE_BLOCK_E];
  __shared__ RankBest rk_wk[RANK ? GATE_WAVES : 1][GATE_ROWS], rk_bn[RANK ? GATE_WAVES : 1][GATE_ROWS];
  __shared__ float rk_wsk[RANK ? GATE_WAVES : 1][GATE_ROWS], rk_wsn[RANK ? GATE_WAVES : 1][GATE_ROWS];
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int xld = a.d + 8;
  bf16_t* Xs = reinterpret_cast<bf16_t*>(dyn);
  uint32_t* sb = reinterpret_cast<uint32_t*>(dyn + (XLDS ? sizeof(bf16_t) * GATE_ROWS * xld : 0));
  // [4][GATE_ROWS][BWD_LD]: dclean hi, dclean lo, draw hi, draw lo
  bf16_t* Ds = reinterpret_cast<bf16_t*>(
      dyn + (((XLDS ? sizeof(bf16_t) * GATE_ROWS * xld : 0) + sizeof(uint32_t) * (size_t)a.E + 15) &
             ~(size_t)15));
  auto dput = [&](int q, int row, int e, float v) {
    const uint32_t hi = cvt_pk_bf16(v, 0.f) << 16;
    const float lo = v - __uint_as_float(hi);
    Ds[((2 * q) * GATE_ROWS + row) * BWD_LD + e] = (bf16_t)(hi >> 16);
    Ds[((2 * q + 1) * GATE_ROWS + row) * BWD_LD + e] = (bf16_t)(cvt_pk_bf16(lo, 0.f) & 0xffffu);
  };
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * GATE_ROWS;
  // the row's rank terms and kept gates' gradients: requested here, placed in
  // LDS once the tile set-up has waited for its own loads
  int4 ri_r{};
  float dhk_r[8];
  if (tid < GATE_ROWS) {
    const int64_t t = min<int64_t>(t0 + tid, a.T - 1);
    if (!RANK) ri_r = reinterpret_cast<const int4*>(a.rinfo)[t];
#pragma unroll
    for (int s = 0; s < 8; ++s) dhk_r[s] = s < a.k ? a.dhk[t * a.k + s] : 0.f;
  }
  for (int i = tid; i < GATE_ROWS * GATE_BLOCK_E / 4; i += GATE_THREADS)
    reinterpret_cast<float4*>(&dhm[0][0])[i] = float4{0.f, 0.f, 0.f, 0.f};
  bw_tile_setup<T, XLDS>(a, sh, sb, Xs, xld);
  if (tid < GATE_ROWS) {  // read back only by this thread
    if (!RANK) ri[tid] = ri_r;
#pragma unroll
    for (int s = 0; s < 8; ++s) dhk[tid][s] = dhk_r[s];
  }
  const bool smooth = NOISY && a.dload != nullptr;
  const int valid = (int)min<int64_t>(GATE_ROWS, a.T - t0);
  for (int blk = 0; blk < a.E; blk += GATE_BLOCK_E) {
    f32x16 cs, ss, hs, rs, es;
    bw_block_scores<T, NOISY, XLDS>(a, sh, Xs, xld, blk, cs, ss, hs, rs, es);
    const int e = blk + w * 32 + (lane & 31);
    if constexpr (RANK)
      rank_in_registers(cs, ss, hs, e, a.E, sb, sh, a.dload, smooth, rk_wk, rk_bn, rk_wsk, rk_wsn, ri,
                        t0, a.T);
    // one thread per row places the row's terms: the kept gates' gradients,
    // then the k-th and (k+1)-th scores' threshold terms added in that order
    auto in_blk = [&](int x) { return x >= blk && x < blk + GATE_BLOCK_E; };
    if (tid < GATE_ROWS) {
      for (int s = 0; s < a.k; ++s) {
        const int x = sh.kle[tid][s];
        if (in_blk(x)) dhm[tid][x - blk] = dhk[tid][s];
      }
      const int4 rw = ri[tid];
      if (in_blk(rw.x)) dhm[tid][rw.x - blk] += __int_as_float(rw.z);
      if (in_blk(rw.y)) dhm[tid][rw.y - blk] += __int_as_float(rw.w);
    }
    __syncthreads();
    float bsum = 0.f;
    if (e < a.E) {
      const uint32_t km = sb[e];
      const float dl = smooth ? a.dload[e] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, lane);
        const bool kept = (km >> row) & 1u;
        const float dh = dhm[row][e - blk];
        float dc = dh;
        if (NOISY) {
          float dsp = dh * es[r];
          if (smooth) {
            const float th = kept ? sh.k1th[row] : sh.kth[row];
            const float isp = rcp_hw(ss[r]);
            const float z = (cs[r] - th) * isp;
            if (z != INFINITY && z != -INFINITY) {
              const float dz = dl * normal_pdf_f(z);
              dc += dz * isp;
              dsp -= dz * z * isp;
            }
          }
          // d softplus(raw) / d raw = sigmoid(raw)
          const float sg = rcp_hw(1.0f + exp2_hw(-rs[r] * 1.4426950408889634f));
          if (row < valid) {
            if (a.draw_hi) split_store(a.draw_hi, a.draw_lo, (t0 + row) * a.E + e, dsp * sg);
            else a.draw[(t0 + row) * a.E + e] = dsp * sg;
          }
          if (DXG) dput(1, row, e, row < valid ? dsp * sg : 0.f);
        }
        if (row < valid) {
          if (a.dclean_hi) split_store(a.dclean_hi, a.dclean_lo, (t0 + row) * a.E + e, dc);
          else a.dclean[(t0 + row) * a.E + e] = dc;
        }
        if (DXG) dput(0, row, e, row < valid ? dc : 0.f);
        bsum += row < valid ? dc : 0.f;
      }
    } else if (DXG) {
      // experts past E: zero k columns of the product
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, lane);
        dput(0, row, e, 0.f);
        if (NOISY) dput(1, row, e, 0.f);
      }
    }
    bsum += __shfl_xor(bsum, 32, 64);
    if (lane < 32 && e < a.E) a.dbias_part[(int64_t)blockIdx.x * a.E + e] = bsum;
    if (blk + GATE_BLOCK_E < a.E) {  // clear the row's entries for the next block
      __syncthreads();
      if (tid < GATE_ROWS) {
        for (int s = 0; s < a.k; ++s) {
          const int x = sh.kle[tid][s];
          if (in_blk(x)) dhm[tid][x - blk] = 0.f;
        }
        const int4 rw = ri[tid];
        if (in_blk(rw.x)) dhm[tid][rw.x - blk] = 0.f;
        if (in_blk(rw.y)) dhm[tid][rw.y - blk] = 0.f;
      }
    }
  }
  if constexpr (DXG) {
    __syncthreads();
    const int w = threadIdx.x >> 6, fr = lane & 31, fh = lane >> 5, q4 = fh * 4;
    const int nks = a.e16 / 16;
    const bf16_t* Dch = Ds;
    const bf16_t* Dcl = Ds + GATE_ROWS * BWD_LD;
    const bf16_t* Drh = Ds + 2 * GATE_ROWS * BWD_LD;
    const bf16_t* Drl = Ds + 3 * GATE_ROWS * BWD_LD;
    // Column blocks cb and cb + GATE_WAVES in one pass: each score-gradient
    // fragment read from LDS feeds both blocks' MFMAs, and the two
    // accumulators are independent chains.  Each block sums its k-steps in
    // the order of the one-block loop (dclean hi, lo, draw hi, lo per step).
    auto store_cols = [&](const f32x16& acc, int cb) {
      // register group g: columns cb*32 + 8g + q4 .. +3 of row fr
      if (fr >= valid || cb * 32 >= a.d) return;
      float* orow = a.dxg + (t0 + fr) * a.d;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c = cb * 32 + 8 * g + q4;
        if (c + 3 < a.d) {
          *reinterpret_cast<float4*>(orow + c) =
              float4{acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]};
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (c + r < a.d) orow[c + r] = acc[4 * g + r];
        }
      }
    };
    for (int cb = w; cb * 32 < a.d; cb += 2 * GATE_WAVES) {
      const int cb2 = cb + GATE_WAVES;
      const int col = cb * 32 + fr, col2 = cb2 * 32 + fr;
      const bool cok = col < a.d, cok2 = col2 < a.d;
      const int64_t o1 = (int64_t)(cok ? col : 0) * a.e16 + 8 * fh;
      const int64_t o2 = (int64_t)(cok2 ? col2 : 0) * a.e16 + 8 * fh;
      f32x16 acc = f32x16{}, acc2 = f32x16{};
      // the tables' fragments of DXG_PF k-steps are requested together
      // (steps past the last re-read the last one and go unused)
      constexpr int DXG_PF = 4;
      for (int ks0 = 0; ks0 < nks; ks0 += DXG_PF) {
        bf16x8 zg[DXG_PF], zg2[DXG_PF], zn[DXG_PF], zn2[DXG_PF];
#pragma unroll
        for (int u = 0; u < DXG_PF; ++u) {
          const int64_t ko = (int64_t)min(ks0 + u, nks - 1) * 16;
          zg[u] = load_bf16x8(a.wgt + o1 + ko);
          zg2[u] = load_bf16x8(a.wgt + o2 + ko);
          if (NOISY) {
            zn[u] = load_bf16x8(a.wnt + o1 + ko);
            zn2[u] = load_bf16x8(a.wnt + o2 + ko);
          }
        }
#pragma unroll
        for (int u = 0; u < DXG_PF; ++u) {
          if (ks0 + u < nks) {
            const int k = (ks0 + u) * 16 + 8 * fh;
            const bf16x8 dch = load_bf16x8(Dch + fr * BWD_LD + k);
            const bf16x8 dcl = load_bf16x8(Dcl + fr * BWD_LD + k);
            acc = mfma32(zg[u], dch, acc);
            acc2 = mfma32(zg2[u], dch, acc2);
            acc = mfma32(zg[u], dcl, acc);
            acc2 = mfma32(zg2[u], dcl, acc2);
            if (NOISY) {
              const bf16x8 drh = load_bf16x8(Drh + fr * BWD_LD + k);
              const bf16x8 drl = load_bf16x8(Drl + fr * BWD_LD + k);
              acc = mfma32(zn[u], drh, acc);
              acc2 = mfma32(zn2[u], drh, acc2);
              acc = mfma32(zn[u], drl, acc);
              acc2 = mfma32(zn2[u], drl, acc2);
            }
          }
        }
      }
      // lanes of columns past d read column 0 of the tables; those columns are not stored
      store_cols(acc, cb);
      store_cols(acc2, cb2);
    }
  }
}

__global__ __launch_bounds__(256) void bw_transpose_table_kernel(const bf16_t* in, int E, int d,
                                                                 int e16, bf16_t* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // out index: c * e16 + e
  if (i >= (int64_t)d * e16) return;
  const int c = (int)(i / e16), e = (int)(i % e16);
  out[i] = e < E ? in[(int64_t)e * d + c] : (bf16_t)0;
}

// out[c] = sum over rows r of part[r][c]: 64 columns per workgroup, wave w
// sums rows w, w+16, ... in order, then the 16 wave sums are added in wave
// order.
__global__ __launch_bounds__(1024) void bw_sum_rows_kernel(const float* part, int64_t nrow,
                                                           int64_t ncol, float* out) {
  __shared__ float ws[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 64 + lane;
  // rows w, w + 16, ... in order, eight loads in flight at a time
  float s = 0.f;
  if (c < ncol) {
    int64_t r = w;
    for (; r + 16 * 7 < nrow; r += 16 * 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = part[(r + 16 * j) * ncol + c];
#pragma unroll
      for (int j = 0; j < 8; ++j) s += v[j];
    }
    for (; r < nrow; r += 16) s += part[r * ncol + c];
  }
  ws[w][lane] = s;
  __syncthreads();
  if (w == 0 && c < ncol) {
    float t = 0.f;
    for (int i = 0; i < 16; ++i) t += ws[i][lane];
    out[c] = t;
  }
}

// out[i] = cast(sum over chunks of part[chunk][i]) in chunk order
template <typename TO>
__global__ __launch_bounds__(256) void bw_sum_chunks_kernel(const float* part, int nchunk,
                                                            int64_t n, TO* out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // eight chunks' loads in flight at a time, added in chunk order
  float s = 0.f;
  int c = 0;
  for (; c + 8 <= nchunk; c += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = part[(int64_t)(c + j) * n + i];
#pragma unroll
    for (int j = 0; j < 8; ++j) s += v[j];
  }
  for (; c < nchunk; ++c) s += part[(int64_t)c * n + i];
  Elem<TO>::store(out, i, s);
}

// out[p][c] = src[perm[p] / k][c] (times scale[perm[p]] when scale is set),
// rounded to the layer's type: the routed rows in expert order, 8 elements
// (bf16) or 4 (fp32) per thread.
template <typename T>
__global__ __launch_bounds__(256) void bw_gather_rows_kernel(const T* src, const int32_t* perm,
                                                             int k, const float* scale, int64_t A,
                                                             int d, T* out) {
  constexpr int V = sizeof(T) == 2 ? 8 : 4;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = d / V;
  if (i >= A * per) return;
  const int64_t p = i / per;
  const int c = (int)(i % per) * V;
  const int a = perm[p];
  const u32x4 v = *reinterpret_cast<const u32x4*>(src + (int64_t)(a / k) * d + c);
  u32x4 o = v;
  if (scale) {
    const float sc = scale[a];
    if constexpr (V == 8) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        o[j] = cvt_pk_bf16(__uint_as_float(v[j] << 16) * sc, __uint_as_float(v[j] & 0xffff0000u) * sc);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = __float_as_uint(__uint_as_float(v[j]) * sc);
    }
  }
  *reinterpret_cast<u32x4*>(out + p * d + c) = o;
}

// dx[t][c] = dx_gate[t][c] + sum_s dxs[inv[t*k+s]][c], slots in order; 16
// bytes of dx per thread (8 bf16 or 4 fp32 columns; d a multiple of that),
// the token's k <= 8 slot positions loaded before the rows
template <typename TO>
__global__ __launch_bounds__(256) void bw_assemble_dx_kernel(const float* dxg, const TO* dxs,
                                                             const int32_t* inv, int64_t T, int k,
                                                             int d, TO* dx, bool vec_out) {
  constexpr int V = 16 / sizeof(TO);
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V;
  if (i >= T * d) return;
  const int64_t t = i / d;
  const int c = (int)(i % d);
  int rows[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) rows[s] = s < k ? inv[t * k + s] : -1;
  float v[V];
#pragma unroll
  for (int j = 0; j < V; j += 4) {
    const float4 q = *reinterpret_cast<const float4*>(dxg + i + j);
    v[j] = q.x;
    v[j + 1] = q.y;
    v[j + 2] = q.z;
    v[j + 3] = q.w;
  }
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (rows[s] < 0) continue;  // no slot, or dropped by a capacity
    const u32x4 raw = *reinterpret_cast<const u32x4*>(dxs + (int64_t)rows[s] * d + c);
    const TO* r = reinterpret_cast<const TO*>(&raw);
#pragma unroll
    for (int j = 0; j < V; ++j) v[j] += Elem<TO>::load(r, j);
  }
  if (vec_out) {
    u32x4 out;
    TO* o = reinterpret_cast<TO*>(&out);
#pragma unroll
    for (int j = 0; j < V; ++j) Elem<TO>::store(o, j, v[j]);
    *reinterpret_cast<u32x4*>(dx + i) = out;
  } else {  // dx not 16-byte aligned
#pragma unroll
    for (int j = 0; j < V; ++j) Elem<TO>::store(dx, i + j, v[j]);
  }
}

// ---------------------------------------------------------------------------
// Products.  C[m][n] = sum_k A(m, k) B(n, k) for each problem (an expert, or
// the single gate problem), operands described by BwOp:
//   kmajor: element (r, k) at p + e*estride + src(r)*ld + k
//   else:   element (r, k) at p + e*estride + src(k)*ld + r
// with src(i) = gather ? gather[i] / gk : i, times scale[gather ? gather[i] :
// i] when scale is set.  Geometry (BwGemm::mode):
//   POS   rows m are the positions of expert e (absolute, offsets[e] ..), K
//         fixed; grid = row tiles of the tile map x column tiles
//   WGT   M, N fixed per expert, k runs over the positions of expert e
//   PLAIN one problem; grid = row tiles x column tiles x K chunks
// ---------------------------------------------------------------------------
constexpr int BG_BM = 128, BG_BN = 128;

__device__ __forceinline__ bool bw_kmajor(const BwOp& o) {
  return o.kind == BW_KB || o.kind == BW_KF;
}
__device__ __forceinline__ float bw_elem(const BwOp& o, int e, int64_t r, int64_t k) {
  const int64_t off = (int64_t)e * o.estride + (bw_kmajor(o) ? r * o.ld + k : k * o.ld + r);
  const bool f32 = o.kind == BW_KF || o.kind == BW_TF;
  return f32 ? ((const float*)o.p)[off] : bf16_to_f32(((const bf16_t*)o.p)[off]);
}

// The part of v an operand carries into a bf16 product: v itself (rounded to
// bf16 by the caller), or with `lo` the residual v - bf16(v), exact in fp32,
// so that a hi pass and a lo pass together carry about 16 significant bits.
__device__ __forceinline__ float bw_part(int lo, float v) {
  if (!lo) return v;
  const uint32_t hi = cvt_pk_bf16(v, 0.f) << 16;
  return v - __uint_as_float(hi);
}

// An LDS operand tile: ROWS rows (128, or 32 for the row operands of small
// experts' tiles) of BK bf16 k values (+8 of padding).
template <int BK, int ROWS = BG_BM>
using BwTileT = bf16_t[ROWS][BK + 8];

// Column of element (row, k) in a tile of a K-major operand (KB, KF).
// Slices swap their 16-byte chunks by row, chunk ^ ((row >> 4) & (BK / 8 -
// 1)), so that the fragment reads of the MFMAs stay free of bank conflicts.
// Every write and read of such a tile goes through this map.
template <int BK>
__device__ __forceinline__ int bw_col(int row, int k) {
  return (((k >> 3) ^ ((row >> 4) & (BK / 8 - 1))) << 3) | (k & 7);
}

// Transposed operands (TB, TF) sit in their tile as stored, [k][128 rows]
// (256 bytes per k, no padding), 16-byte chunks swizzled as chunk ^ 2 (k & 3);
// element (row, k) is at bw_tr_at(k, row).  The MFMA fragments come from
// gfx950's transposing LDS read: within each group of 16 lanes, lane j points
// at k + j / 4, rows r + 4 (j % 4) .. +3, and ds_read_b64_tr_b16 hands lane i
// of the group the four k values of row r + i.  A group's 16 reads touch 8
// distinct chunks, and a wave's 8-byte tile writes fill whole 256-byte k rows,
// so neither conflicts on banks.
typedef short bw_v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ int bw_tr_at(int k, int row) {
  return (k * (BG_BM / 8) + ((row >> 3) ^ (2 * (k & 3)))) * 8 + (row & 7);
}
// fragment of rows r0 .. r0 + 31 (lane l: row r0 + l % 32), k0 + 8 (l / 32) .. +7
__device__ __forceinline__ bf16x8 bw_frag_tr(const bf16_t* T, int r0, int k0) {
  typedef bw_v4i16 __attribute__((address_space(3))) * lds_v4p;
  const int lane = threadIdx.x & 63, G = lane >> 4, j = lane & 15;
  const int r = r0 + 16 * (G & 1) + 4 * (j & 3);
  const int k = k0 + 8 * (G >> 1) + (j >> 2);
  const bw_v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(T + bw_tr_at(k, r)));
  const bw_v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4p)(T + bw_tr_at(k + 4, r)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Loaders of one K slice (BK) of 128 rows of an operand, by kind: load()
// issues the global reads into registers (one slice ahead), put() writes them
// to an LDS tile as bf16 [row][k].  Thread t covers
//   KB, KF: 16-byte k pieces: rows t/(BK/8) + (2048/BK) i, k = (t%(BK/8))*8 .. +7
//   TB, TF: 4-row pieces: rows (t%32)*4 .. +3, k = (t/32)*4 + 32 j .. +3
template <int KIND, int BK, int ROWS = BG_BM> struct BwLd;

// (KB: piece tid + 256 i is row (tid + 256 i) / CPR; with 32 rows and
// 32-wide slices only the first 128 threads hold one)
template <int BK, int ROWS> struct BwLd<BW_KB, BK, ROWS> {
  static constexpr int CPR = BK / 8;                      // pieces per row
  static constexpr int PIECES = ROWS * CPR, NI = (PIECES + 255) / 256;  // per thread
  struct Raw { u32x4 v[NI]; };
  static __device__ __forceinline__ void load(const BwOp& o, int e, int64_t r0, int64_t R,
                                              int64_t k0, int64_t K, Raw& raw) {
    const int tid = threadIdx.x;
    const bf16_t* p = (const bf16_t*)o.p + (int64_t)e * o.estride;
    const int64_t k = k0 + (tid % CPR) * 8;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int piece = tid + 256 * i;
      const int64_t r = r0 + piece / CPR;
      raw.v[i] = (piece < PIECES && r < R && k < K)
                     ? *reinterpret_cast<const u32x4*>(p + r * o.ld + k)
                     : u32x4{0u, 0u, 0u, 0u};
    }
  }
  static __device__ __forceinline__ void put(const BwOp&, const Raw& raw, BwTileT<BK, ROWS>& S) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int piece = tid + 256 * i;
      if (piece >= PIECES) continue;
      const int row = piece / CPR;
      *reinterpret_cast<u32x4*>(&S[row][bw_col<BK>(row, (tid % CPR) * 8)]) = raw.v[i];
    }
  }
};

template <int BK, int ROWS> struct BwLd<BW_TB, BK, ROWS> {
  static_assert(ROWS == BG_BM, "transposed operands fill 128-row tiles");
  static constexpr int NJ = BK / 32;  // 4-k groups per thread
  struct Raw { uint2 v[NJ][4]; };
  static __device__ __forceinline__ void load(const BwOp& o, int e, int64_t r0, int64_t R,
                                              int64_t k0, int64_t K, Raw& raw) {
    const int tid = threadIdx.x;
    const bf16_t* p = (const bf16_t*)o.p + (int64_t)e * o.estride;
    const int64_t r = r0 + (tid & 31) * 4;
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t k = k0 + (tid >> 5) * 4 + 32 * jj + j;
        raw.v[jj][j] = (r < R && k < K) ? *reinterpret_cast<const uint2*>(p + k * o.ld + r)
                                        : uint2{0u, 0u};
      }
  }
  static __device__ __forceinline__ void put(const BwOp&, const Raw& raw, BwTileT<BK>& S) {
    const int tid = threadIdx.x;
    const int rr = (tid & 31) * 4;
    bf16_t* T = &S[0][0];
#pragma unroll
    for (int jj = 0; jj < NJ; ++jj) {
      const int kq = (tid >> 5) * 4 + 32 * jj;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<uint2*>(T + bw_tr_at(kq + j, rr)) = raw.v[jj][j];
    }
  }
};

template <int BK, int ROWS> struct BwLd<BW_KF, BK, ROWS> {
  static_assert(ROWS == BG_BM, "fp32 operands fill 128-row tiles");
  static_assert(BK == 32, "fp32 operands use 32-wide slices");
  struct Raw { float v[2][8]; };
  static __device__ __forceinline__ void load(const BwOp& o, int e, int64_t r0, int64_t R,
                                              int64_t k0, int64_t K, Raw& raw) {
    const int tid = threadIdx.x;
    const float* p = (const float*)o.p + (int64_t)e * o.estride;
    const int64_t k = k0 + (tid & 3) * 8;
    const bool vec = (o.ld & 3) == 0 && k + 8 <= K;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t r = r0 + (tid >> 2) + 64 * i;
      const float* q = p + (r < R ? r : 0) * o.ld + k;
      if (r < R && vec) {
        const float4 a = *reinterpret_cast<const float4*>(q);
        const float4 b = *reinterpret_cast<const float4*>(q + 4);
        raw.v[i][0] = a.x; raw.v[i][1] = a.y; raw.v[i][2] = a.z; raw.v[i][3] = a.w;
        raw.v[i][4] = b.x; raw.v[i][5] = b.y; raw.v[i][6] = b.z; raw.v[i][7] = b.w;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) raw.v[i][j] = (r < R && k + j < K) ? q[j] : 0.f;
      }
    }
  }
  static __device__ __forceinline__ void put(const BwOp& o, const Raw& raw, BwTileT<BK>& S) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      u32x4 out;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        out[j] = cvt_pk_bf16(bw_part(o.lo, raw.v[i][2 * j]), bw_part(o.lo, raw.v[i][2 * j + 1]));
      const int row = (tid >> 2) + 64 * i;
      *reinterpret_cast<u32x4*>(&S[row][bw_col<BK>(row, (tid & 3) * 8)]) = out;
    }
  }
};

template <int BK, int ROWS> struct BwLd<BW_TF, BK, ROWS> {
  static_assert(ROWS == BG_BM, "fp32 operands fill 128-row tiles");
  static_assert(BK == 32, "fp32 operands use 32-wide slices");
  struct Raw { float v[4][4]; };  // [k][row]
  static __device__ __forceinline__ void load(const BwOp& o, int e, int64_t r0, int64_t R,
                                              int64_t k0, int64_t K, Raw& raw) {
    const int tid = threadIdx.x;
    const float* p = (const float*)o.p + (int64_t)e * o.estride;
    const int64_t r = r0 + (tid & 31) * 4, kq = k0 + (tid >> 5) * 4;
    const bool vec = (o.ld & 3) == 0 && r + 4 <= R;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t k = kq + j;
      const float* q = p + (k < K ? k : 0) * o.ld + r;
      if (k < K && vec) {
        const float4 a = *reinterpret_cast<const float4*>(q);
        raw.v[j][0] = a.x; raw.v[j][1] = a.y; raw.v[j][2] = a.z; raw.v[j][3] = a.w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) raw.v[j][c] = (k < K && r + c < R) ? q[c] : 0.f;
      }
    }
  }
  static __device__ __forceinline__ void put(const BwOp& o, const Raw& raw, BwTileT<BK>& S) {
    const int tid = threadIdx.x;
    const int rr = (tid & 31) * 4, kq = (tid >> 5) * 4;
    bf16_t* T = &S[0][0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = cvt_pk_bf16(bw_part(o.lo, raw.v[j][0]), bw_part(o.lo, raw.v[j][1]));
      const uint32_t y = cvt_pk_bf16(bw_part(o.lo, raw.v[j][2]), bw_part(o.lo, raw.v[j][3]));
      *reinterpret_cast<uint2*>(T + bw_tr_at(kq + j, rr)) = uint2{x, y};
    }
  }
};

// Which problem, rows, columns and K range a workgroup covers.
// TD: a transposed bf16 operand loaded straight into LDS (global_load_lds,
// 16 bytes a lane, no staging registers) in the TB layout above: wave w's
// instruction q fills 16-byte slots s = 64 (NQ w + q) + lane, slot s holding
// rows 8 c .. 8 c + 7 of k = s / 16, c = (s % 16) ^ 2 (k & 3).  Positions past
// K and rows past R read a row of zeros (the launcher checks that rows come
// in whole 16-byte pieces).
template <int BK, int ROWS> struct BwLd<BW_TD, BK, ROWS> {
  static_assert(ROWS == BG_BM, "transposed operands fill 128-row tiles");
  struct Raw {};
  static __device__ __forceinline__ void load(const BwOp&, int, int64_t, int64_t, int64_t,
                                              int64_t, Raw&) {}
  static __device__ __forceinline__ void put(const BwOp&, const Raw&, BwTileT<BK>&) {}
  static __device__ __forceinline__ void direct(const BwOp& o, const bf16_t* zero, int e,
                                                int64_t r0, int64_t R, int64_t k0, int64_t K,
                                                BwTileT<BK>& S) {
    constexpr int NQ = BK * BG_BM * 2 / 1024 / 4;  // 1 KB loads per wave
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const bf16_t* p = (const bf16_t*)o.p + (int64_t)e * o.estride;
    bf16_t* T = &S[0][0];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int sl = 64 * (NQ * w + q) + lane;
      const int kl = sl >> 4;
      const int c = (sl & 15) ^ (2 * (kl & 3));
      const int64_t k = k0 + kl, r = r0 + 8 * c;
      const bf16_t* src = (k < K && r < R) ? p + k * o.ld + r : zero + 8 * c;
      __builtin_amdgcn_global_load_lds(src, T + 512 * (NQ * w + q), 16, 0, 0);
    }
  }
};

struct BwTile {
  int e;
  int64_t m0, M;   // rows m0 .. M-1 (absolute positions in POS mode)
  int64_t n0, N;
  int64_t k0, K;   // k range [k0, K) (absolute positions in WGT mode)
  int chunk;
};

template <int BM = BG_BM>
__device__ __forceinline__ bool bw_tile_of(const BwGemm& g, BwTile* t) {
  const int bid = blockIdx.x;
  if (g.mode == BW_POS) {
    const int q = bid / g.ncol, ct = bid % g.ncol;
    const int Q = g.tiles[g.E];
    if (q >= Q) return false;
    int lo = 0, hi = g.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (g.tiles[mid] <= q) lo = mid; else hi = mid - 1;
    }
    t->e = lo;
    t->m0 = g.offsets[lo] + (int64_t)(q - g.tiles[lo]) * BM;
    t->M = g.offsets[lo + 1];
    t->n0 = (int64_t)ct * BG_BN;
    t->N = g.N;
    t->k0 = 0;
    t->K = g.K;
    t->chunk = 0;
  } else if (g.mode == BW_WGT) {
    const int per = g.nrow * g.ncol;
    const int e = bid / per, rem = bid % per;
    t->e = e;
    t->m0 = (int64_t)(rem / g.ncol) * BG_BM;
    t->M = g.M;
    t->n0 = (int64_t)(rem % g.ncol) * BG_BN;
    t->N = g.N;
    t->k0 = g.offsets[e];
    t->K = g.offsets[e + 1];
    t->chunk = 0;
  } else {
    const int per = g.nrow * g.ncol;
    const int c = bid / per, rem = bid % per;
    t->e = 0;
    t->m0 = (int64_t)(rem / g.ncol) * BG_BM;
    t->M = g.M;
    t->n0 = (int64_t)(rem % g.ncol) * BG_BN;
    t->N = g.N;
    t->k0 = (int64_t)c * g.kchunk;
    t->K = min<int64_t>(g.K, t->k0 + g.kchunk);
    t->chunk = c;
  }
  return true;
}

// Output element (m, n) of a plain product.
__device__ __forceinline__ void bw_store(const BwGemm& g, const BwTile& t, int64_t m, int64_t n,
                                         float v) {
  const int64_t i = (int64_t)t.e * g.c_estride + (int64_t)t.chunk * g.c_chunk + m * g.ldc + n;
  if (g.c_f32) ((float*)g.C)[i] = v;
  else ((bf16_t*)g.C)[i] = f32_to_bf16(v);
}

// The expert-hidden epilogue: acc[0] = X W1^T (pre-activation a), acc[1] =
// dY W2 (dHid), acc[2] = X W3^T (SwiGLU b).  ReLU writes Hid = relu(a) and dP
// = dHid * (a > 0); SwiGLU writes Hid = silu(a) b, dA = dHid b silu'(a), dB =
// dHid silu(a).  All [A][N] bf16.
__device__ __forceinline__ void bw_hidden_store(const BwGemm& g, int64_t m, int64_t n, float a,
                                                float dh, float b) {
  const int64_t i = m * g.N + n;
  bf16_t* hid = (bf16_t*)g.C;
  bf16_t* d1 = (bf16_t*)g.C2;
  if (g.epi == BW_EPI_RELU) {
    hid[i] = f32_to_bf16(fmaxf(a, 0.f));
    d1[i] = f32_to_bf16(a > 0.f ? dh : 0.f);
  } else {
    const float sg = 1.0f / (1.0f + expf(-a));
    const float sl = a * sg;
    hid[i] = f32_to_bf16(sl * b);
    d1[i] = f32_to_bf16(dh * b * sg * (1.0f + a * (1.0f - sg)));
    ((bf16_t*)g.C3)[i] = f32_to_bf16(dh * sl);
  }
}

// LDS bytes of the staged output tile: NOUT tiles of 128 x (128 + pad) of
// the output type.
constexpr int BG_CLD_B = BG_BN + 8;   // bf16 row stride
constexpr int BG_CLD_F = BG_BN + 4;   // fp32 row stride

// bf16 MFMA product: BM x 128 tile (BM = 128: four waves of 64 x 64; BM =
// 32, the row-position products of small experts: four waves of 32 x 32), K
// in slices of BK through two LDS buffers: the global loads of slice s+1 are
// in flight during the MFMAs of slice s and land in the other buffer
// afterwards (one barrier per slice).  NPROD products share the tile: plain
// products (NPROD = 1) sum their npair operand pairs into one accumulator,
// the hidden epilogue runs 2 (ReLU) or 3 (SwiGLU) products.  Operand kinds
// are template arguments: KA for every A operand, KB0 for the B operands
// except that of product 1 (KB1).  The results go through LDS and leave as
// 16-byte row pieces.
// (two products in slices of 32: two workgroups per compute unit; 32-row
// tiles hold a quarter of the accumulators and of the row operands' LDS, and
// three share a compute unit)
// NB = 1: one LDS buffer, the next slice written once every wave has read the
// current one (bf16 expert table gradients, whose tiles run one to a few
// slices: the smaller LDS fits three workgroups per compute unit)
template <int NPROD, int KA, int KB0, int KB1, int BK, int NB = 2, int BM = BG_BM>
__global__ __launch_bounds__(256, KA == BW_TD ? 4 : BM == 32 ? 3 : (NPROD == 2 && BK == 32) ? 2 : 1) void
bw_gemm_mfma_kernel(BwGemm g) {
  static_assert(BM == 32 || BM == BG_BM, "tiles of 32 or 128 rows");
  extern __shared__ __attribute__((aligned(16))) bf16_t bw_lds[];
  using TileA = BwTileT<BK, BM>;
  using TileB = BwTileT<BK>;
  // per buffer: the A tiles (A0, and A1 with two or three products: product
  // 2 shares A0), then the B tiles (one per product)
  constexpr int NTA = NPROD == 1 ? 1 : 2, NTB = NPROD;
  constexpr int BUF = NTA * (int)sizeof(TileA) + NTB * (int)sizeof(TileB);
  char* lds_b = reinterpret_cast<char*>(bw_lds);
  auto tA = [&](int buf, int i) -> TileA& {
    return *reinterpret_cast<TileA*>(lds_b + buf * BUF + i * (int)sizeof(TileA));
  };
  auto tB = [&](int buf, int i) -> TileB& {
    return *reinterpret_cast<TileB*>(lds_b + buf * BUF + NTA * (int)sizeof(TileA) +
                                     i * (int)sizeof(TileB));
  };
  BwTile t;
  if (!bw_tile_of<BM>(g, &t)) return;
  // wave grid WM x WN, wave tile RW x CW of MI x NJ 32 x 32 blocks
  constexpr int WM = BM == 32 ? 1 : 2, WN = 4 / WM;
  constexpr int RW = BM / WM, CW = BG_BN / WN, MI = RW / 32, NJ = CW / 32;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w / WN, wn = w % WN, fr = lane & 31, fk = (lane >> 5) * 8;
  using LA = BwLd<KA, BK, BM>;
  using LB0 = BwLd<KB0, BK>;
  using LB1 = BwLd<KB1, BK>;
  f32x16 acc[NPROD][MI][NJ];
#pragma unroll
  for (int p = 0; p < NPROD; ++p)
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[p][i][j] = f32x16{};
  const int64_t nk = (t.K - t.k0 + BK - 1) / BK;
  const int nseg = NPROD == 1 ? g.npair : 1;
  for (int seg = 0; seg < nseg && nk > 0; ++seg) {
    const BwOp& A0 = g.a[seg];
    const BwOp& B0 = g.b[seg];
    const BwOp& A1 = g.a[1];
    const BwOp& B1 = g.b[1];
    const BwOp& B2 = g.b[2];
    typename LA::Raw ra0, ra1;
    typename LB0::Raw rb0, rb2;
    typename LB1::Raw rb1;
    auto load_all = [&](int64_t k0) {
      LA::load(A0, t.e, t.m0, t.M, k0, t.K, ra0);
      LB0::load(B0, t.e, t.n0, t.N, k0, t.K, rb0);
      if constexpr (NPROD >= 2) {
        LA::load(A1, t.e, t.m0, t.M, k0, t.K, ra1);
        LB1::load(B1, t.e, t.n0, t.N, k0, t.K, rb1);
      }
      if constexpr (NPROD == 3) LB0::load(B2, t.e, t.n0, t.N, k0, t.K, rb2);
    };
    // TD (direct) operands are issued with the puts, into their buffer
    auto put_all = [&](int buf, int64_t k0) {
      if constexpr (KA == BW_TD) {
        static_assert(NPROD == 1 && KB0 == BW_TD && NB == 1, "direct loads: one product, one buffer");
        const bf16_t* zero = (const bf16_t*)g.zero;
        LA::direct(A0, zero, t.e, t.m0, t.M, k0, t.K, tA(buf, 0));
        LB0::direct(B0, zero, t.e, t.n0, t.N, k0, t.K, tB(buf, 0));
        return;
      }
      LA::put(A0, ra0, tA(buf, 0));
      LB0::put(B0, rb0, tB(buf, 0));
      if constexpr (NPROD >= 2) {
        LA::put(A1, ra1, tA(buf, 1));
        LB1::put(B1, rb1, tB(buf, 1));
      }
      if constexpr (NPROD == 3) LB0::put(B2, rb2, tB(buf, 2));
    };
    __syncthreads();  // the previous segment's last reads are done
    load_all(t.k0);
    put_all(0, t.k0);
    __syncthreads();
    for (int64_t s = 0; s < nk; ++s) {
      const int cur = NB == 2 ? (int)(s & 1) : 0;
      const int nxt = NB == 2 ? cur ^ 1 : 0;
      const bool more = s + 1 < nk;
      if (more) load_all(t.k0 + (s + 1) * BK);
#pragma unroll
      for (int ks = 0; ks < BK; ks += 16) {
#pragma unroll
        for (int p = 0; p < NPROD; ++p) {
          // product 2 (SwiGLU up) shares product 0's A tile
          const TileA& Ta = tA(cur, p == 2 ? 0 : p);
          const TileB& Tb = tB(cur, p);
          bf16x8 af[MI], bf[NJ];
          // transposed kinds (TB, TF) through the transposing read
          constexpr bool TRA = KA == BW_TB || KA == BW_TF || KA == BW_TD;
          const int KBp = p == 1 ? KB1 : KB0;
          const bool trb = KBp == BW_TB || KBp == BW_TF || KBp == BW_TD;
#pragma unroll
          for (int i = 0; i < MI; ++i) {
            const int ra = wm * RW + i * 32 + fr;
            if constexpr (TRA)
              af[i] = bw_frag_tr(&Ta[0][0], wm * RW + i * 32, ks);
            else
              af[i] = *reinterpret_cast<const bf16x8*>(&Ta[ra][bw_col<BK>(ra, ks + fk)]);
          }
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int rb = wn * CW + j * 32 + fr;
            if (trb)
              bf[j] = bw_frag_tr(&Tb[0][0], wn * CW + j * 32, ks);
            else
              bf[j] = *reinterpret_cast<const bf16x8*>(&Tb[rb][bw_col<BK>(rb, ks + fk)]);
          }
          // B as the first operand: the accumulators hold C^T, so that a lane
          // holds four consecutive columns of one row
#pragma unroll
          for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j) acc[p][i][j] = mfma32(bf[j], af[i], acc[p][i][j]);
        }
      }
      if (more) {
        if constexpr (NB == 1) __syncthreads();  // every wave is done with this buffer
        put_all(nxt, t.k0 + (s + 1) * BK);
      }
      __syncthreads();
    }
  }
  __syncthreads();  // operand tiles free: the output tiles take their place
  // accumulator register r of lane l holds C[row l%32][column 8*(r/4) +
  // 4*(l/32) + r%4] of the wave's (i, j) block: register group g is four
  // consecutive columns of one row
  const int erow = lane & 31, ecol = 4 * (lane >> 5);
  if constexpr (KA == BW_TD) {
    // fp32 partial sums straight from the accumulators, 16 bytes a lane (no
    // LDS staging, which would hold the kernel to two workgroups per CU)
    if (g.c_f32) {
      float* C = (float*)g.C + (int64_t)t.e * g.c_estride + (int64_t)t.chunk * g.c_chunk;
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t m = t.m0 + wm * RW + i * 32 + erow;
            const int64_t n = t.n0 + wn * CW + j * 32 + 8 * q + ecol;
            if (m >= t.M) continue;
            if (n + 3 < t.N) {
              *reinterpret_cast<float4*>(C + m * g.ldc + n) =
                  float4{acc[0][i][j][4 * q], acc[0][i][j][4 * q + 1], acc[0][i][j][4 * q + 2],
                         acc[0][i][j][4 * q + 3]};
            } else {
#pragma unroll
              for (int u = 0; u < 4; ++u)
                if (n + u < t.N) C[m * g.ldc + n + u] = acc[0][i][j][4 * q + u];
            }
          }
      return;
    }
  }
  if constexpr (NPROD == 1) {
    if (g.c_f32) {
      float (*Cs)[BG_CLD_F] = reinterpret_cast<float (*)[BG_CLD_F]>(bw_lds);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(&Cs[wm * RW + i * 32 + erow][wn * CW + j * 32 + 8 * q + ecol]) =
                float4{acc[0][i][j][4 * q], acc[0][i][j][4 * q + 1], acc[0][i][j][4 * q + 2],
                       acc[0][i][j][4 * q + 3]};
      __syncthreads();
      float* C = (float*)g.C + (int64_t)t.e * g.c_estride + (int64_t)t.chunk * g.c_chunk;
      for (int c = tid; c < BM * (BG_BN / 4); c += 256) {
        const int rr = c / (BG_BN / 4), cc = (c % (BG_BN / 4)) * 4;
        const int64_t m = t.m0 + rr, n = t.n0 + cc;
        if (m < t.M && n < t.N)
          *reinterpret_cast<float4*>(C + m * g.ldc + n) = *reinterpret_cast<const float4*>(&Cs[rr][cc]);
      }
    } else {
      bf16_t (*Cs)[BG_CLD_B] = reinterpret_cast<bf16_t (*)[BG_CLD_B]>(bw_lds);
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint2*>(&Cs[wm * RW + i * 32 + erow][wn * CW + j * 32 + 8 * q + ecol]) =
                uint2{cvt_pk_bf16(acc[0][i][j][4 * q], acc[0][i][j][4 * q + 1]),
                      cvt_pk_bf16(acc[0][i][j][4 * q + 2], acc[0][i][j][4 * q + 3])};
      __syncthreads();
      bf16_t* C = (bf16_t*)g.C + (int64_t)t.e * g.c_estride + (int64_t)t.chunk * g.c_chunk;
      for (int c = tid; c < BM * (BG_BN / 8); c += 256) {
        const int rr = c / (BG_BN / 8), cc = (c % (BG_BN / 8)) * 8;
        const int64_t m = t.m0 + rr, n = t.n0 + cc;
        if (m < t.M && n < t.N)
          *reinterpret_cast<u32x4*>(C + m * g.ldc + n) = *reinterpret_cast<const u32x4*>(&Cs[rr][cc]);
      }
    }
  } else {
    // Hid, dP (ReLU) or Hid, dA, dB (SwiGLU), each [A][N] bf16
    constexpr int NOUT = NPROD;
    bf16_t (*Cs)[BM][BG_CLD_B] = reinterpret_cast<bf16_t (*)[BM][BG_CLD_B]>(bw_lds);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int rr = wm * RW + i * 32 + erow, cc = wn * CW + j * 32 + 8 * q + ecol;
          float o0[4], o1[4], o2[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float a = acc[0][i][j][4 * q + u], dh = acc[1][i][j][4 * q + u];
            if constexpr (NPROD == 2) {
              o0[u] = fmaxf(a, 0.f);
              o1[u] = a > 0.f ? dh : 0.f;
              o2[u] = 0.f;
            } else {
              const float b = acc[2][i][j][4 * q + u];
              const float sg = 1.0f / (1.0f + expf(-a));
              const float sl = a * sg;
              o0[u] = sl * b;
              o1[u] = dh * b * sg * (1.0f + a * (1.0f - sg));
              o2[u] = dh * sl;
            }
          }
          *reinterpret_cast<uint2*>(&Cs[0][rr][cc]) =
              uint2{cvt_pk_bf16(o0[0], o0[1]), cvt_pk_bf16(o0[2], o0[3])};
          *reinterpret_cast<uint2*>(&Cs[1][rr][cc]) =
              uint2{cvt_pk_bf16(o1[0], o1[1]), cvt_pk_bf16(o1[2], o1[3])};
          if constexpr (NOUT == 3)
            *reinterpret_cast<uint2*>(&Cs[2][rr][cc]) =
                uint2{cvt_pk_bf16(o2[0], o2[1]), cvt_pk_bf16(o2[2], o2[3])};
        }
    __syncthreads();
    for (int c = tid; c < BM * (BG_BN / 8); c += 256) {
      const int rr = c / (BG_BN / 8), cc = (c % (BG_BN / 8)) * 8;
      const int64_t m = t.m0 + rr, n = t.n0 + cc;
      if (m < t.M && n < t.N) {
        const int64_t o = m * g.N + n;
        *reinterpret_cast<u32x4*>((bf16_t*)g.C + o) = *reinterpret_cast<const u32x4*>(&Cs[0][rr][cc]);
        *reinterpret_cast<u32x4*>((bf16_t*)g.C2 + o) = *reinterpret_cast<const u32x4*>(&Cs[1][rr][cc]);
        if constexpr (NOUT == 3)
          *reinterpret_cast<u32x4*>((bf16_t*)g.C3 + o) = *reinterpret_cast<const u32x4*>(&Cs[2][rr][cc]);
      }
    }
  }
}

// NB = 1 serves bf16 outputs only, so its output tile is bf16 too
template <int NPROD, int BK, int NB = 2, int BM = BG_BM>
static size_t bw_gemm_lds() {
  const int nta = NPROD == 1 ? 1 : 2, ntb = NPROD;
  const size_t ops = sizeof(bf16_t) * NB * (nta * BM + ntb * BG_BM) * (BK + 8);
  const size_t outs = NPROD == 1 && NB == 2 ? sizeof(float) * BM * BG_CLD_F
                                            : sizeof(bf16_t) * NPROD * BM * BG_CLD_B;
  return ops > outs ? ops : outs;
}

// fp32 products: the 128 x 128 tile of the bf16 kernel over 512 threads, K
// in slices of 16 staged through LDS (k-major, padded rows), each thread a
// 4 x 8 block of outputs (rows ty + 32 i, columns tx + 16 j) accumulated with
// fp32 FMA in k order.  The next slice's elements are loaded into registers
// while the current one is multiplied.  NP products share the tile: 1
// (plain: the operand pairs summed in turn), 2 (the ReLU hidden epilogue:
// X W1^T and dY W2) or 3 (SwiGLU: also X W3^T).
constexpr int BF_THREADS = 512, BF_BK = 16, BF_LD = BG_BM + 4;
constexpr int BF_PER = BG_BM * BF_BK / BF_THREADS;  // staged elements per thread and operand

template <int NP>
__global__ __launch_bounds__(BF_THREADS) void bw_gemm_f32_kernel(BwGemm g) {
  constexpr int NOP = NP == 1 ? 2 : NP == 2 ? 4 : 5;  // operands staged per slice
  __shared__ float S[NOP][BF_BK][BF_LD];
  BwTile t;
  if (!bw_tile_of<BG_BM>(g, &t)) return;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  float acc[NP][4][8];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[p][i][j] = 0.f;
  const int64_t nsl = t.K > t.k0 ? (t.K - t.k0 + BF_BK - 1) / BF_BK : 0;
  const int nseg = NP == 1 ? g.npair : 1;
  const int64_t steps = nsl * nseg;
  // operand q of step st: its BwOp and row range (A operands: rows m, B: n)
  auto opq = [&](int64_t st, int q, const BwOp** o, int64_t* rb, int64_t* R) {
    const int seg = NP == 1 ? (int)(st / nsl) : 0;
    const bool isa = NP == 1 ? q == 0 : q < 2;
    *o = NP == 1 ? (q == 0 ? &g.a[seg] : &g.b[seg]) : (q < 2 ? &g.a[q] : &g.b[q - 2]);
    *rb = isa ? t.m0 : t.n0;
    *R = isa ? t.M : t.N;
  };
  float pf[NOP][BF_PER];
  auto fetch = [&](int64_t st) {
    const int64_t k0 = t.k0 + (st % nsl) * BF_BK;
#pragma unroll
    for (int q = 0; q < NOP; ++q) {
      const BwOp* o;
      int64_t rb, R;
      opq(st, q, &o, &rb, &R);
      const bool km = bw_kmajor(*o);
#pragma unroll
      for (int u = 0; u < BF_PER; ++u) {
        const int idx = tid + BF_THREADS * u;
        const int r = km ? idx / BF_BK : idx % BG_BM;
        const int kk = km ? idx % BF_BK : idx / BG_BM;
        const int64_t row = rb + r, k = k0 + kk;
        pf[q][u] = (row < R && k < t.K) ? bw_elem(*o, t.e, row, k) : 0.f;
      }
    }
  };
  auto put = [&](int64_t st) {
#pragma unroll
    for (int q = 0; q < NOP; ++q) {
      const BwOp* o;
      int64_t rb, R;
      opq(st, q, &o, &rb, &R);
      const bool km = bw_kmajor(*o);
#pragma unroll
      for (int u = 0; u < BF_PER; ++u) {
        const int idx = tid + BF_THREADS * u;
        const int r = km ? idx / BF_BK : idx % BG_BM;
        const int kk = km ? idx % BF_BK : idx / BG_BM;
        S[q][kk][r] = pf[q][u];
      }
    }
  };
  if (steps > 0) fetch(0);
  for (int64_t st = 0; st < steps; ++st) {
    put(st);
    __syncthreads();
    if (st + 1 < steps) fetch(st + 1);
#pragma unroll 4
    for (int kk = 0; kk < BF_BK; ++kk) {
      float a0[4], a1[4], b0[8], b1[8], b2[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a0[i] = S[0][kk][ty + 32 * i];
        if (NP > 1) a1[i] = S[1][kk][ty + 32 * i];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        b0[j] = S[NP == 1 ? 1 : 2][kk][tx + 16 * j];
        if (NP > 1) b1[j] = S[3][kk][tx + 16 * j];
        if (NP == 3) b2[j] = S[NOP - 1][kk][tx + 16 * j];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          acc[0][i][j] = fmaf(a0[i], b0[j], acc[0][i][j]);
          if (NP > 1) acc[1][i][j] = fmaf(a1[i], b1[j], acc[1][i][j]);
          if (NP == 3) acc[NP - 1][i][j] = fmaf(a0[i], b2[j], acc[NP - 1][i][j]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t m = t.m0 + ty + 32 * i, n = t.n0 + tx + 16 * j;
      if (m >= t.M || n >= t.N) continue;
      if (NP == 1) {
        bw_store(g, t, m, n, acc[0][i][j]);
        continue;
      }
      const float a = acc[0][i][j], dh = acc[1][i][j];
      const int64_t o = m * g.N + n;
      float* hid = (float*)g.C;
      float* d1 = (float*)g.C2;
      if (NP == 2) {
        hid[o] = fmaxf(a, 0.f);
        d1[o] = a > 0.f ? dh : 0.f;
      } else {
        const float b = acc[NP - 1][i][j];
        const float sg = 1.0f / (1.0f + expf(-a));
        hid[o] = a * sg * b;
        d1[o] = dh * b * sg * (1.0f + a * (1.0f - sg));
        ((float*)g.C3)[o] = dh * a * sg;
      }
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_bw_cv2_grad(const float* imp, const float* load, int E, float wi, float wl,
                              float* dimp, float* dload, hipStream_t s) {
  hipLaunchKernelGGL(bw_cv2_grad_kernel, dim3(1), dim3(256), 0, s, imp, load, E, wi, wl, dimp,
                     dload);
  return hipGetLastError();
}

hipError_t launch_bw_gate_out(const BwGateOutArgs& a, bool bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.T + 3) / 4));
  if (bf16) hipLaunchKernelGGL(bw_gate_out_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(bw_gate_out_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bw_hier_gate(const BwHierGateArgs& a, bool bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.k > 8 || a.kpg <= 0 || a.k % a.kpg != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.T + 3) / 4));
  if (bf16) hipLaunchKernelGGL(bw_hier_gate_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(bw_hier_gate_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bw_expert_rowsum(const BwRowSumArgs& a, bool bf16, hipStream_t s) {
  if (a.E == 0 || a.d == 0) return hipSuccess;
  const dim3 grid((unsigned)a.E, (unsigned)((a.d + 255) / 256));
  if (bf16) hipLaunchKernelGGL(bw_expert_rowsum_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(bw_expert_rowsum_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

static size_t bw_gate_lds(bool xlds, int d, int E, bool dxg = false) {
  const size_t base = (xlds ? sizeof(bf16_t) * GATE_ROWS * (d + 8) : 0) + sizeof(uint32_t) * (size_t)E;
  return dxg ? ((base + 15) & ~(size_t)15) + BWD_LDS : base;
}

int bw_fused_dxg_max_experts() { return GATE_BLOCK_E; }

hipError_t launch_bw_transpose_table(const void* in, int E, int d, int e16, void* out,
                                     hipStream_t s) {
  const int64_t n = (int64_t)d * e16;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(bw_transpose_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     (const bf16_t*)in, E, d, e16, (bf16_t*)out);
  return hipGetLastError();
}

template <typename K>
static hipError_t bw_set_lds(K kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

template <typename T, bool NOISY, bool XLDS>
static hipError_t launch_bw_gate_v(const BwGateArgs& a, hipStream_t s) {
  const size_t lds = bw_gate_lds(XLDS, a.d, a.E);
  const bool one = a.E <= GATE_BLOCK_E;
  hipError_t err = bw_set_lds(bw_gate_rank_kernel<T, NOISY, XLDS>, lds);
  if (err != hipSuccess) return err;
  constexpr bool can_dxg = sizeof(T) == 2;
  const bool dxg = can_dxg && one && a.dxg != nullptr;
  const size_t lds_g = bw_gate_lds(XLDS, a.d, a.E, dxg);
  err = dxg ? bw_set_lds(bw_gate_grad_kernel<T, NOISY, XLDS, can_dxg>, lds_g)
            : bw_set_lds(bw_gate_grad_kernel<T, NOISY, XLDS, false>, lds_g);
  if (err != hipSuccess) return err;
  const dim3 grid((unsigned)((a.T + GATE_ROWS - 1) / GATE_ROWS));
  if (one) {
    // one expert block: the rank step runs inside the gradient kernel
    err = dxg ? bw_set_lds(bw_gate_grad_kernel<T, NOISY, XLDS, can_dxg, true>, lds_g)
              : bw_set_lds(bw_gate_grad_kernel<T, NOISY, XLDS, false, true>, lds_g);
    if (err != hipSuccess) return err;
    if (dxg)
      hipLaunchKernelGGL((bw_gate_grad_kernel<T, NOISY, XLDS, can_dxg, true>), grid,
                         dim3(GATE_THREADS), lds_g, s, a);
    else
      hipLaunchKernelGGL((bw_gate_grad_kernel<T, NOISY, XLDS, false, true>), grid,
                         dim3(GATE_THREADS), lds_g, s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((bw_gate_rank_kernel<T, NOISY, XLDS>), grid, dim3(GATE_THREADS), lds, s, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (dxg)
    hipLaunchKernelGGL((bw_gate_grad_kernel<T, NOISY, XLDS, can_dxg>), grid, dim3(GATE_THREADS),
                       lds_g, s, a);
  else
    hipLaunchKernelGGL((bw_gate_grad_kernel<T, NOISY, XLDS, false>), grid, dim3(GATE_THREADS),
                       lds_g, s, a);
  return hipGetLastError();
}

size_t bw_gate_lds_bytes(bool bf16, int d, int E) {
  return bw_gate_lds(bf16 && d <= GATE_XLDS_MAX_D, d, E);
}

hipError_t launch_bw_gate(const BwGateArgs& a, bool bf16, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  const bool noisy = a.w_noise != nullptr;
  if (bf16) {
    if (a.d <= GATE_XLDS_MAX_D)
      return noisy ? launch_bw_gate_v<bf16_t, true, true>(a, s)
                   : launch_bw_gate_v<bf16_t, false, true>(a, s);
    return noisy ? launch_bw_gate_v<bf16_t, true, false>(a, s)
                 : launch_bw_gate_v<bf16_t, false, false>(a, s);
  }
  return noisy ? launch_bw_gate_v<float, true, false>(a, s)
               : launch_bw_gate_v<float, false, false>(a, s);
}

hipError_t launch_bw_sum_rows(const float* part, int64_t nrow, int64_t ncol, float* out,
                              hipStream_t s) {
  if (ncol == 0) return hipSuccess;
  hipLaunchKernelGGL(bw_sum_rows_kernel, dim3((unsigned)((ncol + 63) / 64)), dim3(1024), 0, s,
                     part, nrow, ncol, out);
  return hipGetLastError();
}

hipError_t launch_bw_sum_chunks(const float* part, int nchunk, int64_t n, bool bf16, void* out,
                                hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bf16) hipLaunchKernelGGL(bw_sum_chunks_kernel<bf16_t>, grid, dim3(256), 0, s, part, nchunk, n, (bf16_t*)out);
  else hipLaunchKernelGGL(bw_sum_chunks_kernel<float>, grid, dim3(256), 0, s, part, nchunk, n, (float*)out);
  return hipGetLastError();
}

hipError_t launch_bw_assemble_dx(const float* dxg, const void* dxs, const int32_t* inv, int64_t T,
                                 int k, int d, bool bf16, void* dx, hipStream_t s) {
  const int V = bf16 ? 8 : 4;  // columns per thread
  if (d % V != 0 || k > 8) return hipErrorInvalidValue;
  const int64_t n = T * d / V;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  const bool vec_out = (reinterpret_cast<uintptr_t>(dx) & 15) == 0;
  if (bf16)
    hipLaunchKernelGGL(bw_assemble_dx_kernel<bf16_t>, grid, dim3(256), 0, s, dxg,
                       (const bf16_t*)dxs, inv, T, k, d, (bf16_t*)dx, vec_out);
  else
    hipLaunchKernelGGL(bw_assemble_dx_kernel<float>, grid, dim3(256), 0, s, dxg,
                       (const float*)dxs, inv, T, k, d, (float*)dx, vec_out);
  return hipGetLastError();
}

hipError_t launch_bw_gather_rows(const void* src, const int32_t* perm, int k, const float* scale,
                                 int64_t A, int d, bool bf16, void* out, hipStream_t s) {
  const int V = bf16 ? 8 : 4;
  const int64_t n = A * (d / V);
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL(bw_gather_rows_kernel<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)src, perm, k, scale, A, d, (bf16_t*)out);
  else
    hipLaunchKernelGGL(bw_gather_rows_kernel<float>, grid, dim3(256), 0, s, (const float*)src, perm, k, scale, A, d, (float*)out);
  return hipGetLastError();
}

int bw_pos_tile_rows(bool bf16, int64_t A, int E) {
  return bf16 && A <= 32 * (int64_t)E ? 32 : BG_BM;
}

template <int NPROD, int KA, int KB0, int KB1, int BK, int NB = 2, int BM = BG_BM>
static hipError_t launch_bw_mfma(const BwGemm& g, int64_t grid, hipStream_t s) {
  auto kern = bw_gemm_mfma_kernel<NPROD, KA, KB0, KB1, BK, NB, BM>;
  const size_t lds = bw_gemm_lds<NPROD, BK, NB, BM>();
  hipError_t err = bw_set_lds(kern, lds);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(256), lds, s, g);
  return hipGetLastError();
}

hipError_t launch_bw_gemm(BwGemm g, bool bf16, int64_t grid, hipStream_t s) {
  g.ncol = (int)((g.N + BG_BN - 1) / BG_BN);
  g.nrow = (int)((g.M + BG_BM - 1) / BG_BM);
  if (grid <= 0 || g.ncol == 0) return hipSuccess;
  if (!bf16) {
    // fp32 products take fp32 operands whole: no hi / lo halves
    for (int i = 0; i < g.npair; ++i)
      if (g.a[i].lo || g.b[i].lo) return hipErrorInvalidValue;
    const dim3 blk(BF_THREADS);
    if (g.epi == BW_EPI_RELU)
      hipLaunchKernelGGL(bw_gemm_f32_kernel<2>, dim3((unsigned)grid), blk, 0, s, g);
    else if (g.epi == BW_EPI_SWIGLU)
      hipLaunchKernelGGL(bw_gemm_f32_kernel<3>, dim3((unsigned)grid), blk, 0, s, g);
    else
      hipLaunchKernelGGL(bw_gemm_f32_kernel<1>, dim3((unsigned)grid), blk, 0, s, g);
    return hipGetLastError();
  }
  if (g.mode == BW_POS && g.pos_rows != BG_BM) {
    // 32-row tiles of the row-position products (experts averaging at most
    // 32 rows): bf16 rows against 128 columns of a table
    if (g.pos_rows != 32) return hipErrorInvalidValue;
    if (g.epi == BW_EPI_RELU) return launch_bw_mfma<2, BW_KB, BW_KB, BW_TB, 32, 2, 32>(g, grid, s);
    if (g.epi == BW_EPI_SWIGLU) return launch_bw_mfma<3, BW_KB, BW_KB, BW_TB, 32, 2, 32>(g, grid, s);
    if (g.a[0].kind != BW_KB || g.b[0].kind != BW_TB) return hipErrorInvalidValue;
    return launch_bw_mfma<1, BW_KB, BW_TB, BW_TB, 64, 2, 32>(g, grid, s);
  }
  // slices of 32: the two products' operand tiles take 80 KB of LDS and at
  // most 256 registers, so that two workgroups share a compute unit (the
  // table gradients, with K over an expert's few rows, keep slices of 64:
  // twice the slices per tile made them slower)
  if (g.epi == BW_EPI_RELU) return launch_bw_mfma<2, BW_KB, BW_KB, BW_TB, 32>(g, grid, s);
  if (g.epi == BW_EPI_SWIGLU) return launch_bw_mfma<3, BW_KB, BW_KB, BW_TB, 32>(g, grid, s);
  const int ka = g.a[0].kind, kb = g.b[0].kind;
  if (kb != BW_TB) return hipErrorInvalidValue;
  switch (ka) {
    case BW_KB: return launch_bw_mfma<1, BW_KB, BW_TB, BW_TB, 64>(g, grid, s);
    case BW_TB:
      // bf16 expert table gradients and the fp32 partial sums of the
      // gate-table products: one LDS buffer (experts that reach this kernel
      // average under 256 rows, so a table-gradient tile runs a few K
      // slices), and operand rows straight into LDS when they come in whole,
      // aligned 16-byte pieces (no staging registers: four workgroups per
      // compute unit; otherwise three for the table gradients)
      if ((g.mode == BW_WGT && !g.c_f32) || (g.mode == BW_PLAIN && g.c_f32 && g.ldc % 4 == 0 &&
                                              ((uintptr_t)g.C & 15) == 0)) {
        bool direct = g.zero && g.M % 8 == 0 && g.N % 8 == 0 && ((uintptr_t)g.zero & 15) == 0;
        for (int i = 0; i < g.npair && direct; ++i)
          direct = g.a[i].kind == BW_TB && g.b[i].kind == BW_TB && !g.a[i].lo && !g.b[i].lo &&
                   g.a[i].ld % 8 == 0 && g.b[i].ld % 8 == 0 && g.a[i].estride % 8 == 0 &&
                   g.b[i].estride % 8 == 0 &&
                   (((uintptr_t)g.a[i].p | (uintptr_t)g.b[i].p) & 15) == 0;
        if (direct) return launch_bw_mfma<1, BW_TD, BW_TD, BW_TD, 64, 1>(g, grid, s);
        if (g.mode == BW_WGT) return launch_bw_mfma<1, BW_TB, BW_TB, BW_TB, 64, 1>(g, grid, s);
      }
      return launch_bw_mfma<1, BW_TB, BW_TB, BW_TB, 64>(g, grid, s);
    case BW_KF: return launch_bw_mfma<1, BW_KF, BW_TB, BW_TB, 32>(g, grid, s);
    default: return launch_bw_mfma<1, BW_TF, BW_TB, BW_TB, 32>(g, grid, s);
  }
}

}  // namespace moe
