// Per-batch equal-size expert mask and its threshold form, in place of
// KeepTopK.
//
// Method ("Outrageously Large Neural Networks: The Sparsely-Gated
// Mixture-of-Experts Layer - 中文验证版", ai-papers.xuzou.cn, section 方法适配):
// in some translation runs a per-batch mask gives every expert the same batch
// size during training, and per-expert thresholds approximate that mask at
// inference.  Read here as:
//   batch mask:      expert e keeps the m tokens of the batch with the
//                    largest noisy scores H[:, e] (ties: the lower token);
//   threshold mask:  expert e keeps every token with H[t, e] >= theta[e], the
//                    first m of them in token order taking rows;
//   gates:           per token, the softmax over the scores of the experts
//                    that kept it ("MoE:稀疏门控混合专家", section 三: softmax
//                    over the kept scores); a token kept by no expert has
//                    no gates and y = 0.
//
//   mask_scores_kernel   H of every (token, expert) with the gate's own
//                        projection code (gate_common.h), written
//                        expert-major Ht[e][t]; the threshold mask's keep
//                        bits straight from the registers
//   mask_select_kernel   batch mask, one workgroup per expert: the m-th best
//                        score of the column by a radix select over
//                        order-preserving keys, then the keep bits, ties at
//                        the cut to the lower tokens
//   (route.hip: counts, per-block ranks and the rows, tokens ascending)
//   mask_token_kernel    per token: the softmax statistics over the experts
//                        that kept it and the number of its pairs with a row
//   mask_scan_kernel     slot offsets of the tokens
//   mask_slots_kernel    per token, experts ascending: expert, gate, row
//   combine_csr_kernel   y_t = sum over the token's slots of gate * y_sorted[row]
//   mask_balance_kernel  per expert: importance (the gates recomputed from
//                        the token statistics, tokens ascending) and load
//                        (the kept count before the cap)
// Every reduction runs in a fixed order, so results are bitwise repeatable.
#include "gate_common.h"
#include "moe_kernels.h"

namespace moe {

// ---------------------------------------------------------------------------
// Scores.  Workgroup = 32 tokens x all experts in blocks of 256, the gate's
// tile geometry: lane l of wave w holds expert blk + 32w + l%32 for the 16
// rows acc_row(i, l), which are four runs of four consecutive rows, written
// to Ht as four 16-byte stores.
// ---------------------------------------------------------------------------
template <typename T, bool NOISY, bool XLDS>
__global__ __launch_bounds__(GATE_THREADS) void mask_scores_kernel(MaskArgs a) {
  __shared__ int rows[GATE_ROWS];
  extern __shared__ __attribute__((aligned(16))) char dyn[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t0 = (int64_t)blockIdx.x * GATE_ROWS;
  const int valid = (int)min<int64_t>(GATE_ROWS, a.T - t0);
  if (tid < GATE_ROWS) rows[tid] = (int)min<int64_t>(t0 + tid, a.T - 1);
  const int xld = a.d + 8;
  bf16_t* Xs = reinterpret_cast<bf16_t*>(dyn);
  __syncthreads();
  if (XLDS) load_x_tile((const bf16_t*)a.x, a.d, rows, GATE_ROWS, Xs, xld);
  __syncthreads();
  const TileX<T> tx{(const T*)a.x, rows, XLDS ? Xs : nullptr, xld};
  const GateTabs tb{a.w_gate, a.w_noise, 0, (const bf16_t*)a.w_pack, 0, a.pack_nt};
  for (int blk = 0; blk < a.E; blk += GATE_BLOCK_E) {
    const int e = blk + w * 32 + (lane & 31);
    const bool ev = e < a.E;
    float ep[16];
    if (NOISY) {
      a.noise.rows16(0, 1, e, a.E, [&](int r) { return rows[acc_row(r, lane)]; }, ep);
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) ep[r] = 0.f;
    }
    f32x16 ac[1], ar[1];
    BlockProj<T, NOISY, XLDS, 1>::run(tx, a.d, tb, blk, a.E, ac, ar);
    const float b = (a.bias && ev) ? a.bias[e] : 0.f;
    float h[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float c = ac[0][r] + b;
      h[r] = select_score(NOISY ? noisy_score(c, ep[r], softplus_f(ar[0][r])) : c);
    }
    if (ev) {
      float* dst = a.Ht + (int64_t)e * a.Tp + t0 + 4 * (lane >> 5);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(dst + 8 * g) =
            make_float4(h[4 * g], h[4 * g + 1], h[4 * g + 2], h[4 * g + 3]);
    }
    if (a.theta) {
      // keep bits of the 32 rows: each half-wave holds 16 of them
      const float th = ev ? a.theta[e] : 0.f;
      uint32_t mine = 0u;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = acc_row(r, lane);
        if (ev && row < valid && h[r] >= th) mine |= 1u << row;
      }
      const uint32_t word = mine | (uint32_t)__shfl_xor((int)mine, 32, 64);
      if (ev && lane < 32) a.bits[(int64_t)blockIdx.x * a.E + e] = word;
    }
  }
}

template <typename T, bool NOISY, bool XLDS>
static hipError_t launch_scores_v(const MaskArgs& a, hipStream_t s) {
  const size_t sh = XLDS ? sizeof(bf16_t) * GATE_ROWS * (size_t)(a.d + 8) : 0;
  static bool attr = false;
  if (sh > 32768 && !attr) {
    hipError_t err = hipFuncSetAttribute((const void*)mask_scores_kernel<T, NOISY, XLDS>,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
    if (err != hipSuccess) return err;
    attr = true;
  }
  hipLaunchKernelGGL((mask_scores_kernel<T, NOISY, XLDS>), dim3(a.NB), dim3(GATE_THREADS), sh, s,
                     a);
  return hipGetLastError();
}

hipError_t launch_mask_scores(const MaskArgs& a, bool bf16, bool noisy, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (bf16) {
    if (a.d <= GATE_XLDS_MAX_D)
      return noisy ? launch_scores_v<bf16_t, true, true>(a, s)
                   : launch_scores_v<bf16_t, false, true>(a, s);
    return noisy ? launch_scores_v<bf16_t, true, false>(a, s)
                 : launch_scores_v<bf16_t, false, false>(a, s);
  }
  return noisy ? launch_scores_v<float, true, false>(a, s)
               : launch_scores_v<float, false, false>(a, s);
}

// ---------------------------------------------------------------------------
// Batch mask.  Keys order the scores as unsigned integers (larger key =
// larger score; -0 is taken as +0, so that equal scores give equal keys).
// Four passes of 8 bits find the key of the m-th best token; `want` is then
// how many of the tokens holding exactly that key are kept, lowest first.
// ---------------------------------------------------------------------------
constexpr int SEL_THREADS = 256;

__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(SEL_THREADS) void mask_select_kernel(MaskArgs a) {
  __shared__ int hist[SEL_THREADS / 64][256];  // one histogram per wave
  __shared__ int s_digit, s_want;
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* col = a.Ht + (int64_t)e * a.Tp;
  const int T = (int)a.T;
  uint32_t prefix = 0u, pmask = 0u;
  int want = min(a.m, T);
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < (SEL_THREADS / 64) * 256; i += SEL_THREADS) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += SEL_THREADS) {
      const uint32_t k = order_key(col[t]);
      if ((k & pmask) == prefix) atomicAdd(&hist[w][(k >> shift) & 255], 1);
    }
    __syncthreads();
    if (w == 0) {
      // lane l holds digits 255 - 4l .. 252 - 4l, the largest first
      int c[4], sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dg = 255 - 4 * lane - j;
        int v = 0;
#pragma unroll
        for (int q = 0; q < SEL_THREADS / 64; ++q) v += hist[q][dg];
        c[j] = v;
        sum += v;
      }
      const int incl = wave_incl_scan(sum);
      const int excl = incl - sum;
      if (excl < want && incl >= want) {
        int run = excl;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (run < want && run + c[j] >= want) {
            s_digit = 255 - 4 * lane - j;
            s_want = want - run;
          }
          run += c[j];
        }
      }
    }
    __syncthreads();
    prefix |= (uint32_t)s_digit << shift;
    pmask |= 255u << shift;
    want = s_want;
    __syncthreads();
  }
  // keep bits: thread i takes a contiguous run of 32-token blocks, and the
  // tokens holding the cut key are ranked in token order across threads
  const int per = (a.NB + SEL_THREADS - 1) / SEL_THREADS;
  const int b0 = min(a.NB, tid * per), b1 = min(a.NB, b0 + per);
  int neq = 0;
  for (int b = b0; b < b1; ++b)
    for (int j = 0; j < 32; ++j) {
      const int t = 32 * b + j;
      if (t < T && order_key(col[t]) == prefix) ++neq;
    }
  int total;
  int eqr = block_excl_scan<SEL_THREADS>(neq, &total);
  for (int b = b0; b < b1; ++b) {
    uint32_t word = 0u;
    for (int j = 0; j < 32; ++j) {
      const int t = 32 * b + j;
      if (t >= T) break;
      const uint32_t k = order_key(col[t]);
      if (k > prefix) {
        word |= 1u << j;
      } else if (k == prefix) {
        if (eqr < want) word |= 1u << j;
        ++eqr;
      }
    }
    a.bits[(int64_t)b * a.E + e] = word;
  }
}

hipError_t launch_mask_select(const MaskArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  hipLaunchKernelGGL(mask_select_kernel, dim3(a.E), dim3(SEL_THREADS), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Tokens: one wave per token.  Lane l looks at experts l, l + 64, ...: the
// token's bit in bits[b][e], its rank among e's kept tokens (base plus the
// kept tokens before it in the block) and, when kept, its score Ht[e][t].
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__global__ __launch_bounds__(256) void mask_token_kernel(MaskArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const int64_t b = t >> 5;
  const uint32_t bit = 1u << (t & 31);
  const uint32_t* word = a.bits + b * a.E;
  const int32_t* base = a.base + b * a.E;
  float mx = -INFINITY;
  for (int e = lane; e < a.E; e += 64)
    if (word[e] & bit) mx = fmaxf(mx, a.Ht[(int64_t)e * a.Tp + t]);
  mx = wave_max_f(mx);
  float sum = 0.f;
  int rows = 0;
  for (int e = lane; e < a.E; e += 64) {
    const uint32_t wd = word[e];
    if (wd & bit) {
      sum += expf(a.Ht[(int64_t)e * a.Tp + t] - mx);
      const int rank = base[e] + __popc(wd & (bit - 1u));
      if (rank < a.m) ++rows;
    }
  }
  sum = wave_sum(sum);
  rows = wave_sum(rows);
  if (lane == 0) {
    a.tokstat[t] = make_float2(mx, sum > 0.f ? 1.0f / sum : 0.f);
    a.nslot[t] = rows;
  }
}

// Exclusive scan of the slot counts into tok_off[0..T] (one workgroup).
constexpr int MSCAN_THREADS = 1024;
__global__ __launch_bounds__(MSCAN_THREADS) void mask_scan_kernel(MaskArgs a) {
  const int64_t T = a.T;
  const int64_t per = (T + MSCAN_THREADS - 1) / MSCAN_THREADS;
  const int64_t t0 = min<int64_t>(T, threadIdx.x * per), t1 = min<int64_t>(T, t0 + per);
  int sum = 0;
  for (int64_t t = t0; t < t1; ++t) sum += a.nslot[t];
  int total;
  int run = block_excl_scan<MSCAN_THREADS>(sum, &total);
  for (int64_t t = t0; t < t1; ++t) {
    a.tok_off[t] = run;
    run += a.nslot[t];
  }
  if (threadIdx.x == 0) a.tok_off[T] = total;
}

__global__ __launch_bounds__(256) void mask_slots_kernel(MaskArgs a) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= a.T) return;
  const int64_t b = t >> 5;
  const uint32_t bit = 1u << (t & 31);
  const uint32_t* word = a.bits + b * a.E;
  const int32_t* base = a.base + b * a.E;
  const float2 st = a.tokstat[t];
  const int64_t j0 = a.tok_off[t];
  int written = 0;
  for (int e0 = 0; e0 < a.E; e0 += 64) {
    const int e = e0 + lane;
    bool has = false;
    int pos = 0;
    float g = 0.f;
    if (e < a.E) {
      const uint32_t wd = word[e];
      if (wd & bit) {
        const int rank = base[e] + __popc(wd & (bit - 1u));
        if (rank < a.m) {
          has = true;
          pos = a.offsets[e] + rank;
          g = expf(a.Ht[(int64_t)e * a.Tp + t] - st.x) * st.y;
        }
      }
    }
    const uint64_t bal = __ballot(has);
    if (has) {
      const int64_t j = j0 + written + __popcll(bal & ((1ull << lane) - 1ull));
      a.slot_e[j] = e;
      a.slot_g[j] = g;
      a.slot_pos[j] = pos;
    }
    written += __popcll(bal);
  }
}

hipError_t launch_mask_tokens(const MaskArgs& a, hipStream_t s) {
  if (a.T == 0) {
    hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(MSCAN_THREADS), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)((a.T + 3) / 4));
  hipLaunchKernelGGL(mask_token_kernel, grid, dim3(256), 0, s, a);
  hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(MSCAN_THREADS), 0, s, a);
  hipLaunchKernelGGL(mask_slots_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Combine over the token's slots, ascending, fp32 accumulation; one wave per
// token, 16-byte column chunks when the row allows.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void combine_csr_kernel(const T* __restrict__ ys,
                                                          const int32_t* __restrict__ tok_off,
                                                          const int32_t* __restrict__ slot_pos,
                                                          const float* __restrict__ slot_g,
                                                          int64_t Tn, int d, T* __restrict__ y) {
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= Tn) return;
  constexpr int V = 16 / sizeof(T);
  const int j0 = tok_off[t], j1 = tok_off[t + 1];
  if (d % V == 0) {
    for (int c = lane * V; c < d; c += 64 * V) {
      float acc[V];
#pragma unroll
      for (int i = 0; i < V; ++i) acc[i] = 0.f;
      for (int j = j0; j < j1; ++j) {
        const float g = slot_g[j];
        u32x4 raw = *reinterpret_cast<const u32x4*>(ys + (int64_t)slot_pos[j] * d + c);
        const T* vals = reinterpret_cast<const T*>(&raw);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = fmaf(g, Elem<T>::load(vals, i), acc[i]);
      }
      u32x4 out;
      T* ov = reinterpret_cast<T*>(&out);
#pragma unroll
      for (int i = 0; i < V; ++i) Elem<T>::store(ov, i, acc[i]);
      *reinterpret_cast<u32x4*>(y + t * d + c) = out;
    }
  } else {
    for (int c = lane; c < d; c += 64) {
      float acc = 0.f;
      for (int j = j0; j < j1; ++j)
        acc = fmaf(slot_g[j], Elem<T>::load(ys, (int64_t)slot_pos[j] * d + c), acc);
      Elem<T>::store(y, t * d + c, acc);
    }
  }
}

hipError_t launch_combine_csr(const void* y_sorted, const int32_t* tok_off,
                              const int32_t* slot_pos, const float* slot_g, int64_t T, int d,
                              bool bf16, void* y, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + 3) / 4));
  if (bf16)
    hipLaunchKernelGGL(combine_csr_kernel<bf16_t>, grid, dim3(256), 0, s,
                       (const bf16_t*)y_sorted, tok_off, slot_pos, slot_g, T, d, (bf16_t*)y);
  else
    hipLaunchKernelGGL(combine_csr_kernel<float>, grid, dim3(256), 0, s, (const float*)y_sorted,
                       tok_off, slot_pos, slot_g, T, d, (float*)y);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Balance statistics, one workgroup per expert: thread i walks a contiguous
// run of 32-token blocks, tokens ascending, adding the gate of every token
// the expert kept (recomputed from the token's statistics: the same
// operations as its slot gate) and counting them; the 256 partial sums are
// added by a fixed butterfly per wave, then the four waves in order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void mask_balance_kernel(MaskArgs a) {
  __shared__ float ws[4];
  __shared__ int wc[4];
  const int e = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (a.NB + 255) / 256;
  const int b0 = min(a.NB, tid * per), b1 = min(a.NB, b0 + per);
  const float* col = a.Ht + (int64_t)e * a.Tp;
  float s = 0.f;
  int n = 0;
  for (int b = b0; b < b1; ++b) {
    uint32_t wd = a.bits[(int64_t)b * a.E + e];
    n += __popc(wd);
    while (wd) {
      const int i = __ffs(wd) - 1;
      wd &= wd - 1u;
      const int64_t t = 32 * (int64_t)b + i;
      const float2 st = a.tokstat[t];
      s += expf(col[t] - st.x) * st.y;
    }
  }
  s = wave_sum(s);
  n = wave_sum(n);
  if (lane == 0) {
    ws[w] = s;
    wc[w] = n;
  }
  __syncthreads();
  if (tid == 0) {
    a.importance[e] = ((ws[0] + ws[1]) + ws[2]) + ws[3];
    a.load[e] = (float)(wc[0] + wc[1] + wc[2] + wc[3]);
  }
}

hipError_t launch_mask_balance(const MaskArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(mask_balance_kernel, dim3(a.E), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
