// Fast Walsh-Hadamard transform of a chunk held in LDS: radix-8 register
// passes over bit ranges of the flat element index (Sylvester order, no
// normalisation). Shared by the BiIP passes and the inference transforms.
#pragma once
#include <hip/hip_runtime.h>

namespace kq {

// LDS index with one pad word per 32 elements (spreads the strided passes
// over the banks)
__device__ __host__ constexpr int padi(int i) { return i + (i >> 5); }


__device__ inline void bfly8(float v[8], int nb) {
  // nb radix-2 stages over the 3-bit register index (nb <= 3)
#pragma unroll
  for (int s = 0; s < 3; ++s) {
    if (s >= nb) break;
    const int h = 1 << s;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j & h) continue;
      const float a = v[j], b = v[j + h];
      v[j] = a + b;
      v[j + h] = a - b;
    }
  }
}

// Butterflies over bits [bit_lo, bit_lo + nbits) of the flat LDS index, for a
// chunk of n_el (power of two) elements. Radix-8 register passes.
__device__ inline void lds_fwht(float* s, int n_el, int bit_lo, int nbits) {
  const int t = threadIdx.x;
  for (int q = bit_lo; q < bit_lo + nbits; q += 3) {
    const int nb = min(3, bit_lo + nbits - q);
    const int span = 1 << nb;
    const int ngroups = n_el >> nb;
    for (int g = t; g < ngroups; g += blockDim.x) {
      const int base = ((g >> q) << (q + nb)) | (g & ((1 << q) - 1));
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < span) v[j] = s[padi(base + (j << q))];
      bfly8(v, nb);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < span) s[padi(base + (j << q))] = v[j];
    }
    __syncthreads();
  }
}

// One radix-2^NB pass over bits [Q, Q + NB) of the flat LDS index with Q and
// NB known at compile time. A group's base has those bits clear and its
// offsets J = j << Q use only them, so padi(base + J) = padi(base) + J +
// (J >> 5): every access is the base plus a constant.
template <int Q, int NB>
__device__ inline void lds_fwht_pass_ct(float* s, int n_el) {
  const int ngroups = n_el >> NB;
  for (int g = threadIdx.x; g < ngroups; g += blockDim.x) {
    const int base = ((g >> Q) << (Q + NB)) | (g & ((1 << Q) - 1));
    float* p = s + padi(base);
    float v[8];
#pragma unroll
    for (int j = 0; j < (1 << NB); ++j) v[j] = p[(j << Q) + ((j << Q) >> 5)];
    bfly8(v, NB);
#pragma unroll
    for (int j = 0; j < (1 << NB); ++j) p[(j << Q) + ((j << Q) >> 5)] = v[j];
  }
  __syncthreads();
}

// Butterflies over bits [0, LGB), radix 8 (the last pass narrower).
template <int LGB, int Q = 0>
__device__ inline void lds_fwht_ct(float* s, int n_el) {
  if constexpr (Q < LGB) {
    constexpr int NB = LGB - Q < 3 ? LGB - Q : 3;
    lds_fwht_pass_ct<Q, NB>(s, n_el);
    lds_fwht_ct<LGB, Q + NB>(s, n_el);
  }
}

// Butterflies over bits [0, lgb): the compile-time passes for LGB > 0 (then
// lgb must equal LGB), the generic ones for LGB = 0.
template <int LGB>
__device__ inline void lds_fwht_blk(float* s, int n_el, int lgb) {
  if constexpr (LGB > 0) lds_fwht_ct<LGB>(s, n_el);
  else lds_fwht(s, n_el, 0, lgb);
}

}  // namespace kq
