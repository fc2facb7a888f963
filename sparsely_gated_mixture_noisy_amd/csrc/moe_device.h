// Device-side helpers shared by the HIP kernels of the MoE layer (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // storage type of bfloat16 values in memory
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) {
  return __uint_as_float(((uint32_t)v) << 16);
}

// float -> bfloat16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Two floats -> two bfloat16 (round to nearest even) in one dword, low half
// first: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// 16-byte vector load of 8 bf16 values as the MFMA operand type.
__device__ __forceinline__ bf16x8 load_bf16x8(const bf16_t* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  u32x4 v = {0u, 0u, 0u, 0u};
  return __builtin_bit_cast(bf16x8, v);
}

// D(32x32, fp32) += A(32x16) * B(16x32); operands bf16.
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32];
// accumulator register r of lane l holds D[8*(r/4) + 4*(l/32) + r%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x32) * B(32x16); operands bf16.
// Lane l supplies A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16];
// accumulator register r of lane l holds D[4*(l/16) + r][l%16].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Hardware 2^x and log2(x) (v_exp_f32 / v_log_f32, about 1 ulp).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float rcp_hw(float x) { return __builtin_amdgcn_rcpf(x); }

// softplus(z) = ln(1 + e^z) = max(z, 0) + ln(1 + u), u = e^-|z| in (0, 1].
// ln(1 + u) is taken as ln(y) - ((y - 1) - u) / y with y = fl(1 + u), which
// cancels the rounding of 1 + u (the classic compensated log1p).
__device__ __forceinline__ float softplus_f(float z) {
  constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
  const float u = exp2_hw(-fabsf(z) * kLog2e);
  const float y = 1.0f + u;
  const float lp = log2_hw(y) * kLn2 - ((y - 1.0f) - u) * rcp_hw(y);
  return fmaxf(z, 0.0f) + lp;
}

// erfc(x) by the Chebyshev fit of Press, Teukolsky, Vetterling and Flannery
// (Numerical Recipes, 2nd ed., section 6.2, "erfcc"): fractional error below
// 1.2e-7 for every x.
__device__ __forceinline__ float erfc_f(float x) {
  const float ax = fabsf(x);
  const float t = rcp_hw(1.0f + 0.5f * ax);
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  const float r = t * exp2_hw((p - ax * ax) * 1.4426950408889634f);
  return x >= 0.0f ? r : 2.0f - r;
}

// Standard normal CDF: Phi(z) = erfc(-z / sqrt 2) / 2.
__device__ __forceinline__ float normal_cdf_f(float z) {
  return 0.5f * erfc_f(-z * 0.70710678118654752440f);
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

// Ranking of gate candidates: larger score first, lower expert index on ties.
__device__ __forceinline__ bool ranks_before(float v1, int e1, float v2, int e2) {
  return v1 > v2 || (v1 == v2 && e1 < e2);
}

// Sum over the 64 lanes of a wave by a fixed xor butterfly (offsets 32 .. 1):
// every lane ends with the same bits, and the order does not depend on
// scheduling.
template <typename F>
__device__ __forceinline__ F wave_sum(F v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (integers).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

// Rows of tile i of the nt tiles that hold an expert's m rows: the
// ceil(m / 32) blocks of 32 rows go to the tiles as evenly as possible, whole
// blocks first, so the tiles run no more MFMA row blocks than the rows need
// (near-equal row counts would give 130 rows two tiles of three blocks).
__device__ __forceinline__ void tile_rows(int m, int nt, int i, int* first, int* rows) {
  const int nblk = (m + 31) / 32, base = nblk / nt, rem = nblk % nt;
  const int b0 = i * base + min(i, rem), nb = base + (i < rem ? 1 : 0);
  *first = 32 * b0;
  *rows = min(m, 32 * (b0 + nb)) - 32 * b0;
}

// Exclusive prefix sum of one int per thread over a workgroup of NT threads
// (NT a multiple of 64); *total gets the sum.  One barrier pair.
template <int NT>
__device__ int block_excl_scan(int v, int* total) {
  __shared__ int wsum[NT / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int x = wsum[i];
    if (i < w) base += x;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return base + incl - v;
}

// Sum of 256 slot values held by threads 0..255 of a workgroup of NT >= 256
// threads: a butterfly inside each of the first four waves, then
// (w0 + w1) + (w2 + w3).  The order is a function of the slots only, so any
// NT gives the same bits.
template <int NT>
__device__ double sum256_f64(double v) {
  static_assert(NT >= 256 && NT % 64 == 0, "needs the first four waves");
  __shared__ double ws[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (w < 4) {
    const double x = wave_sum(v);
    if (lane == 0) ws[w] = x;
  }
  __syncthreads();
  const double r = (ws[0] + ws[1]) + (ws[2] + ws[3]);
  __syncthreads();
  return r;
}

// Squared coefficient of variation of v[0..E): population variance / mean^2
// in fp64 (0 when the mean is 0).  Slot i < 256 sums v[i], v[i+256], ... in
// order; the slots are added by sum256_f64.  Called by all NT threads.
// A slot's values are loaded eight at a time, so that their loads are in
// flight together; the sums keep the order above.
template <int NT>
__device__ double cv2_of(const float* v, int E) {
  const int tid = threadIdx.x;
  double s = 0.0;
  if (tid < 256) {
    int i = tid;
    for (; i + 7 * 256 < E; i += 8 * 256) {
      float u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = v[i + j * 256];
#pragma unroll
      for (int j = 0; j < 8; ++j) s += (double)u[j];
    }
    for (; i < E; i += 256) s += (double)v[i];
  }
  const double mean = sum256_f64<NT>(s) / E;
  double q = 0.0;
  if (tid < 256) {
    int i = tid;
    for (; i + 7 * 256 < E; i += 8 * 256) {
      float u[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) u[j] = v[i + j * 256];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const double dv = (double)u[j] - mean;
        q += dv * dv;
      }
    }
    for (; i < E; i += 256) {
      const double dv = (double)v[i] - mean;
      q += dv * dv;
    }
  }
  const double var = sum256_f64<NT>(q) / E;
  return mean == 0.0 ? 0.0 : var / (mean * mean);
}

// Map a linear workgroup id to a tile id so that consecutive tile ids land on
// the same XCD (workgroups are dispatched round-robin over the 8 XCDs) and are
// dispatched close in time; tiles of one expert then share that XCD's L2.
__device__ __forceinline__ int xcd_tile_id(int bid, int grid) {
  const int nx = 8;
  int per = (grid + nx - 1) / nx;
  int x = bid % nx, slot = bid / nx;
  return x * per + slot;
}

}  // namespace moe
