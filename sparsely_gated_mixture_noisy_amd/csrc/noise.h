// Noise of the noisy gate ("MoE:稀疏门控混合专家", nengyongai.cn, section 四:
// a fresh standard-normal draw per call), either read from a caller tensor
// or drawn inside the kernels from a counter-based generator.
//
// Generator: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC 2011) over a 128-bit counter with a
// 64-bit key (the caller's seed); ten rounds, each multiplying counter words
// 0 and 2 by two fixed constants, mixing the high halves with words 1 and 3
// and the round key, the key bumped by two Weyl constants after each round.
// Element j of the noise row of token t (group g of the hierarchy's
// secondary noise, else 0; stream 0 for the flat and secondary noise, 1 for
// the primary) takes counter (j / 4, t, g, stream): output words (0, 1) give
// elements 4q and 4q+1, words (2, 3) elements 4q+2 and 4q+3, by the
// Box-Muller transform r = sqrt(-2 ln u_a), r cos(2 pi u_b) (even element)
// or r sin(2 pi u_b) (odd), u = (top 23 bits + 1/2) / 2^23 (exact in fp32).
// The draw of an element depends on its indices only, never on the launch.
#pragma once
#include "moe_device.h"

namespace moe {

constexpr uint32_t PHILOX_M0 = 0xD2511F53u, PHILOX_M1 = 0xCD9E8D57u;
constexpr uint32_t PHILOX_W0 = 0x9E3779B9u, PHILOX_W1 = 0xBB67AE85u;

__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t lo0 = PHILOX_M0 * c[0], hi0 = __umulhi(PHILOX_M0, c[0]);
    const uint32_t lo1 = PHILOX_M1 * c[2], hi1 = __umulhi(PHILOX_M1, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
}

// (top 23 bits of x + 1/2) / 2^23, exact in fp32, in (0, 1)
__device__ __forceinline__ float uniform23(uint32_t x) {
  return ((float)(x >> 9) + 0.5f) * 0x1p-23f;
}


// The four normals of one Philox call: elements 4q .. 4q+3 of a noise row.
__device__ __forceinline__ void noise_quad(uint32_t q, uint32_t t, uint32_t g, uint32_t stream,
                                           uint32_t k0, uint32_t k1, float (&z)[4]) {
  uint32_t c[4] = {q, t, g, stream};
  philox4x32_10(c, k0, k1);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const float r = sqrtf(-2.0f * logf(uniform23(c[2 * p])));
    const float ub = uniform23(c[2 * p + 1]);
    z[2 * p] = r * cospif(2.0f * ub);
    z[2 * p + 1] = r * sinpif(2.0f * ub);
  }
}

// Value of lane (quad base + J) for every lane of its quad.
template <int J>
__device__ __forceinline__ float quad_bcast(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), J * 0x55, 0xF, 0xF, false));
}

// One element: the same arithmetic as the quad.
__device__ __forceinline__ float noise_normal(uint32_t j, uint32_t t, uint32_t g, uint32_t stream,
                                              uint32_t k0, uint32_t k1) {
  float z[4];
  noise_quad(j >> 2, t, g, stream, k0, k1, z);
  return z[j & 3u];
}

// Where a kernel takes its noise from: a tensor, or the generator.
struct NoiseSrc {
  const float* eps = nullptr;  // [T][G][n] (flat and primary: G = 1), when gen == 0
  uint32_t k0 = 0, k1 = 0;     // key: the seed's low and high words
  int gen = 0;
  int stream = 0;              // 0: flat / secondary noise, 1: primary
  __host__ __device__ bool on() const { return gen != 0 || eps != nullptr; }
  // element j of the n-element noise row of token t, group g of G
  __device__ __forceinline__ float at(int64_t t, int g, int G, int j, int n) const {
    if (gen) return noise_normal((uint32_t)j, (uint32_t)t, (uint32_t)g, (uint32_t)stream, k0, k1);
    return eps[((int64_t)t * G + g) * n + j];
  }
  // The noise of 16 rows for the calling lane's element j (group g of G, row
  // length n), row r of the 16 being token tok(r).  With the generator, the
  // four lanes of each quad must hold elements 4q .. 4q+3 of the same rows
  // (tok(r) equal across the quad) and call this together: lane q4 of the
  // quad draws rows r = 4m + q4 (one Philox call and two Box-Muller pairs
  // each) and hands every lane its element through the quad.  Elements j >=
  // n are drawn but the caller must ignore them.
  template <typename TokF>
  __device__ __forceinline__ void rows16(int g, int G, int j, int n, TokF tok,
                                         float (&out)[16]) const {
    if (!gen) {
#pragma unroll
      for (int r = 0; r < 16; ++r) out[r] = j < n ? eps[((int64_t)tok(r) * G + g) * n + j] : 0.f;
      return;
    }
    const int q4 = threadIdx.x & 3;
    float mine[4][4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      noise_quad((uint32_t)(j >> 2), (uint32_t)tok(4 * m + q4), (uint32_t)g, (uint32_t)stream, k0,
                 k1, mine[m]);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = r >> 2;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x;
        if ((r & 3) == 0) x = quad_bcast<0>(mine[m][e]);
        else if ((r & 3) == 1) x = quad_bcast<1>(mine[m][e]);
        else if ((r & 3) == 2) x = quad_bcast<2>(mine[m][e]);
        else x = quad_bcast<3>(mine[m][e]);
        v[e] = x;
      }
      out[r] = q4 == 0 ? v[0] : q4 == 1 ? v[1] : q4 == 2 ? v[2] : v[3];
    }
  }
};

}  // namespace moe
