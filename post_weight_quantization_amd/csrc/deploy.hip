// Inference with a quantized layer: packed codes and the product with the
// layer in its original basis.
//
// KronQ explainer (gist.science), "Limitazioni": the only inference overhead
// is the orthogonal transforms. The sweep quantizes W' = U S_G W S_X V^T, so
//   y = W^ x = S_G^-1 U^T (W^' (V (S_X^-1 x))),
// with U = blockdiag(H_b / sqrt b) diag(sign_out) and V likewise on the input
// side. One call is three launches:
//   1. transform_in: x2 = V S_X^-1 x, a row FWHT in LDS with sign_in / s_x
//      folded into the load, written out per 32-value chunk in the form the
//      product reads (below);
//   2. qmatvec: y1 = W^' x2 straight from the packed codes. The columns are
//      cut into K tiles of 2048 (64 lanes x one 32-code chunk each). A
//      workgroup owns a run of rows and its waves share out the K tiles; a
//      lane keeps its chunk of x2 in registers for all of the rows and
//      decodes each row's codes into sum_k q_k x_k. With 128-column groups
//      the chunk's grid applies at once, scale (sum q x - zero sum x); with
//      one grid per row it applies to the row's total, scale (sum_j q_j x_j
//      - zero sum_j x_j), after the workgroup's sums meet. Per-row
//      sums over the 64 lanes go through a transposing butterfly (8 rows x
//      NB vectors leave the wave in 10 shuffles for NB = 1); the waves'
//      sums meet in LDS and are added in wave order (no atomics);
//   3. transform_out: FWHT of each output block of y1, then sign_out / s_g
//      and 1 / sqrt(b).
// 2-bit codes with one grid per row (d_in a multiple of 512: the workloads'
// setting) take the matrix-core path further down: the codes are fp4
// operands of v_mfma_scale_f32_16x16x128_f8f6f4 as they stand and the input
// enters as fp8 digits with E8M0 block scales. The rest:
// Products: for 2-, 4- and 8-bit codes in integers. Each chunk of x2 is held
// in fixed point against its own largest magnitude: with 2^(e-1) <=
// max |x_k| < 2^e, m_k = rint(x_k 2^(22 - e)), |m_k| <= 2^22, and x_k =
// m_k 2^(e - 22) up to half a unit of 2^(e - 22), below fp32's rounding of
// the chunk's largest value. m_k is split into signed limbs, and a packed
// word under a field mask lines its codes up with the limbs of one limb
// word, so one dot instruction sums several products exactly in int32:
//   2- and 4-bit codes: six 4-bit limbs (m = sum_l n_l 16^l, n_l in
//     [-8, 7]), dot8 over 8 codes; 4-bit codes enter as q - 8 to fit a
//     signed nibble. The limbs are taken from the top down, the sum shifted
//     by 4 bits between them (|sum q m| < 2^30: exact);
//   8-bit codes: three byte limbs (m = l0 + 2^8 l1 + 2^16 l2), dot4 over 4
//     codes entered as q - 128, the limb sums combined in fp32.
// That is 24 dot instructions per 32 codes and vector, against 2
// conversions and fused multiply-adds per code in fp32. 3-bit codes
// straddle words and use fp32 products (bit-field extract, conversion,
// fused multiply-add).
// Packing: code j of a row in bits [b j, b j + b) of a little-endian stream
// of 32-bit words, rows padded to a multiple of 4 words.
#include "kq_internal.h"
#include "fwht_lds.h"

#include <type_traits>
#include <utility>

namespace kq {

namespace {

constexpr int LANES = 64;
constexpr int CODES = 32;   // codes of a row per lane and K tile: one chunk
constexpr int XW = 32;      // words per chunk and vector of the prepared input
constexpr int G = 8;        // rows per group: G x NB values reduced together
constexpr int SLOT = 64;    // rows x vectors per workgroup of the product
constexpr int TCH = 8192;   // elements per LDS transform chunk
constexpr int TCHP = TCH + TCH / 32;

// Prepared chunk (XW words). Integer products: words 0-23 hold the limbs,
// limb l of 2- and 4-bit codes in words 4 l .. 4 l + 3, of 8-bit codes in
// words 8 l .. 8 l + 7. Limb word j of a limb holds in field f (nibble or
// byte) the limb of the code that field f of the masked packed word j
// holds: 2-bit codes, word j = 2 i + p <- packed word i shifted by 2 p,
// nibble f = code 16 i + 2 f + p; 4-bit codes, nibble f of word j = code
// 8 j + f; 8-bit codes, byte f of word j = code 4 j + f. Word 24 =
// 2^(e - 22) and word 25 = sum m_k as floats. fp32 products: the 32 values.
constexpr int W_UNIT = 24, W_MSUM = 25;

// The integer products take codes q - offset: signed nibbles for 4-bit
// codes, signed bytes for 8-bit codes.
__device__ constexpr float code_offset(int bits) { return bits == 4 ? 8.f : bits == 8 ? 128.f : 0.f; }


__global__ void pack_kernel(const uint8_t* __restrict__ codes, int64_t d_out, int64_t d_in, int bits,
                            int64_t row_words, uint32_t* __restrict__ packed) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= d_out * row_words) return;
  const int64_t row = e / row_words, w = e % row_words;
  const int64_t b0 = 32 * w;
  int64_t j0 = b0 / bits;
  const int64_t j1 = min(d_in - 1, (b0 + 31) / bits);
  uint32_t v = 0;
  for (int64_t j = j0; j <= j1; ++j) {
    const uint32_t c = codes[row * d_in + j];
    const int64_t sh = int64_t(bits) * j - b0;
    v |= sh >= 0 ? (c << sh) : (c >> (-sh));
  }
  packed[e] = v;
}

inline int ilog2(int64_t v) {
  int k = 0;
  while ((int64_t(1) << (k + 1)) <= v) ++k;
  return k;
}

// Launch helper: f(std::integral_constant<int, LGB>) with the transforms'
// FWHT passes fixed at compile time for the workloads' 4096 and 8192 blocks
// (LGB = 12, 13), generic otherwise (LGB = 0).
template <class F>
void with_lgb(int lgb, F&& f) {
  if (lgb == 12) f(std::integral_constant<int, 12>{});
  else if (lgb == 13) f(std::integral_constant<int, 13>{});
  else f(std::integral_constant<int, 0>{});
}

// Transform chunk: the largest L with blk | L, L | n, L <= TCH.
int64_t transform_len(int64_t n, int64_t blk) {
  int64_t L = blk;
  while (L * 2 <= TCH && n % (L * 2) == 0) L *= 2;
  return L;
}

// x2 = gain * H_blk (x[b] sign_in / s_x) over a chunk of L = 2^lgL columns
// of vector b, written as prepared chunks xq[b][c] (XW words each). One
// workgroup per chunk of columns; blockDim is a multiple of 64 dividing L
// (or 64 when L = 32).
template <int BITS, int LGB>
__global__ __launch_bounds__(1024) void transform_in_kernel(const float* __restrict__ x, int64_t d_in,
                                                            int lgL, int lgb,
                                                            const int8_t* __restrict__ si,
                                                            const float* __restrict__ s_x, float gain,
                                                            uint32_t* __restrict__ xq) {
  __shared__ float s[TCHP];
  const int L = 1 << lgL;
  const int64_t per_row = d_in >> lgL;
  const int64_t b = blockIdx.x / per_row;
  const int64_t c0 = int64_t(blockIdx.x % per_row) << lgL;
  const float* src = x + b * d_in + c0;
  for (int e = 4 * threadIdx.x; e < L; e += 4 * blockDim.x) {
    const float4 v = *reinterpret_cast<const float4*>(src + e);
    const float4 sx = *reinterpret_cast<const float4*>(s_x + c0 + e);
    s[padi(e)] = v.x * float(si[c0 + e]) / sx.x;
    s[padi(e + 1)] = v.y * float(si[c0 + e + 1]) / sx.y;
    s[padi(e + 2)] = v.z * float(si[c0 + e + 2]) / sx.z;
    s[padi(e + 3)] = v.w * float(si[c0 + e + 3]) / sx.w;
  }
  __syncthreads();
  lds_fwht_blk<LGB>(s, L, lgb);
  const int64_t nchunk = d_in / CODES;
  uint32_t* dst = xq + (b * nchunk + (c0 >> 5)) * XW;  // this chunk's first prepared chunk
  if constexpr (BITS == 3) {
    for (int e = threadIdx.x; e < L; e += blockDim.x) dst[e] = __float_as_uint(gain * s[padi(e)]);
  } else {
    constexpr bool NIB = BITS != 8;
    constexpr int NL = NIB ? 6 : 3, LB = NIB ? 4 : 8;  // limbs, bits per limb
    __shared__ int8_t lim[TCH * 6];
    __shared__ float meta[TCH / CODES][2];
    // one value per lane; the 32 lanes of a half-wave hold one chunk
    for (int e = threadIdx.x; e < L; e += blockDim.x) {
      const float v = gain * s[padi(e)];
      float mx = fabsf(v);
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
      int ex = 0;
      if (mx > 0.f) frexpf(mx, &ex);  // mx = f 2^ex, 1/2 <= f < 1
      const int m = int(rintf(ldexpf(v, 22 - ex)));
      int r = m;
#pragma unroll
      for (int l = 0; l < NL; ++l) {
        const int h = 1 << (LB - 1);
        const int n = ((r + h) & (2 * h - 1)) - h;  // balanced digit
        lim[e * 6 + l] = int8_t(n);
        r = (r - n) >> LB;
      }
      int ms = m;
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) ms += __shfl_xor(ms, o);
      if ((e & (CODES - 1)) == 0) {
        meta[e >> 5][0] = ldexpf(1.f, ex - 22);
        meta[e >> 5][1] = float(ms);
      }
    }
    __syncthreads();
    // one output word per thread: chunk e / 32, word e % 32
    for (int e = threadIdx.x; e < L; e += blockDim.x) {
      const int ch = e >> 5, j = e & 31;
      uint32_t word = 0u;
      if (j < 24) {
        const int l = NIB ? j >> 2 : j >> 3, wi = NIB ? j & 3 : j & 7;
        constexpr int FIELDS = NIB ? 8 : 4;
#pragma unroll
        for (int f = 0; f < FIELDS; ++f) {
          const int k = BITS == 2 ? 16 * (wi >> 1) + 2 * f + (wi & 1) : BITS == 4 ? 8 * wi + f : 4 * wi + f;
          const uint32_t digit = uint32_t(int(lim[(32 * ch + k) * 6 + l])) & ((1u << LB) - 1);
          word |= digit << (LB * f);
        }
      } else if (j == W_UNIT) {
        word = __float_as_uint(meta[ch][0]);
      } else if (j == W_MSUM) {
        word = __float_as_uint(meta[ch][1]);
      }
      dst[e] = word;
    }
  }
}

// y[b][r0 + e] = gain * sign_out / s_g * (H_blk y1[b])[r0 + e]
// where y1 is the sum of `planes` partial planes, `plane` floats apart,
// added in plane order
template <int LGB>
__global__ __launch_bounds__(1024) void transform_out_kernel(const float* __restrict__ y1,
                                                             int64_t d_out, int lgL, int lgb,
                                                             const int8_t* __restrict__ so,
                                                             const float* __restrict__ s_g, float gain,
                                                             int planes, int64_t plane,
                                                             float* __restrict__ y) {
  __shared__ float s[TCHP];
  const int L = 1 << lgL;
  const int64_t per_row = d_out >> lgL;
  const int64_t b = blockIdx.x / per_row;
  const int64_t r0 = int64_t(blockIdx.x % per_row) << lgL;
  const float* src = y1 + b * d_out + r0;
  for (int e = 4 * threadIdx.x; e < L; e += 4 * blockDim.x) {
    float4 v = *reinterpret_cast<const float4*>(src + e);
    for (int p = 1; p < planes; ++p) {
      const float4 u = *reinterpret_cast<const float4*>(src + p * plane + e);
      v.x += u.x;
      v.y += u.y;
      v.z += u.z;
      v.w += u.w;
    }
    s[padi(e)] = v.x;
    s[padi(e + 1)] = v.y;
    s[padi(e + 2)] = v.z;
    s[padi(e + 3)] = v.w;
  }
  __syncthreads();
  lds_fwht_blk<LGB>(s, L, lgb);
  float* dst = y + b * d_out + r0;
  for (int e = threadIdx.x; e < L; e += blockDim.x)
    dst[e] = gain * s[padi(e)] * float(so[r0 + e]) / s_g[r0 + e];
}

// One step of the transposing butterfly over v[0 .. 2H): lanes with bit o
// set keep the upper half, the others the lower, and each adds the half its
// partner keeps. Constant indices only, so the values stay in registers.
template <int N, int H, int... I>
__device__ inline void fold_step(float (&v)[N], int lane, int o, std::integer_sequence<int, I...>) {
  const bool up = lane & o;
  ((v[I] = (up ? v[I + H] : v[I]) + __shfl_xor(up ? v[I] : v[I + H], o)), ...);
}

// Sums of N values (N a power of two <= 64) over the 64 lanes: transposing
// steps at offsets 32, 16, ... leave lane L with value L >> (6 - log2 N)
// summed over its 64 / N neighbours, plain steps finish the sum.
template <int N, int K = 0>
__device__ inline float fold_all(float (&v)[N], int lane) {
  if constexpr ((N >> K) >= 2) {
    fold_step<N, (N >> (K + 1))>(v, lane, 32 >> K, std::make_integer_sequence<int, (N >> (K + 1))>{});
    return fold_all<N, K + 1>(v, lane);
  } else {
    float t = v[0];
#pragma unroll
    for (int o = 32 >> K; o > 0; o >>= 1) t += __shfl_xor(t, o);
    return t;
  }
}

// The codes of one row's chunk (p in bounds: lanes past the last chunk read
// the last chunk, and their input chunk is zero)
template <int BITS>
__device__ inline void load_codes(const uint32_t* p, uint32_t (&w)[BITS]) {
  if constexpr (BITS == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    w[0] = v.x;
    w[1] = v.y;
  } else if constexpr (BITS == 4 || BITS == 8) {
#pragma unroll
    for (int h = 0; h < BITS / 4; ++h) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[h];
      w[4 * h] = v.x;
      w[4 * h + 1] = v.y;
      w[4 * h + 2] = v.z;
      w[4 * h + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < BITS; ++i) w[i] = p[i];
  }
}

// Codes of one group of G rows for this lane's chunk: rows past `last`
// repeat row `last` (in bounds; their values are not stored).
template <int BITS, int G>
__device__ inline void load_group(const uint32_t* gp, int rw, int last, uint32_t (&wc)[G][BITS]) {
#pragma unroll
  for (int r = 0; r < G; ++r) load_codes<BITS>(gp + min(r, last) * rw, wc[r]);
}

// sum_k q_k x_k of every row of a group and vector, pr[r][b]. The rows'
// dependency chains are interleaved (row index innermost), so consecutive
// instructions are independent.
template <int BITS, int NB>
__device__ inline void group_dot(const uint32_t (&wc)[G][BITS], const uint32_t (&xw)[NB][XW],
                                 float (&pr)[G][NB]) {
  if constexpr (BITS == 2 || BITS == 4) {
    // nibble masks of the packed words (4-bit codes as q - 8) against the
    // nibble limb words, top limb first, shifting the sums by 4 bits
    // between limbs
    uint32_t t[G][4];
#pragma unroll
    for (int r = 0; r < G; ++r) {
      if constexpr (BITS == 2) {
        t[r][0] = wc[r][0] & 0x33333333u;
        t[r][1] = (wc[r][0] >> 2) & 0x33333333u;
        t[r][2] = wc[r][1] & 0x33333333u;
        t[r][3] = (wc[r][1] >> 2) & 0x33333333u;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) t[r][i] = wc[r][i] ^ 0x88888888u;
      }
    }
    int d[G][NB];
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) d[r][b] = 0;
#pragma unroll
    for (int l = 5; l >= 0; --l) {
      if (l < 5) {
#pragma unroll
        for (int r = 0; r < G; ++r)
#pragma unroll
          for (int b = 0; b < NB; ++b) d[r][b] <<= 4;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < G; ++r)
            d[r][b] = __builtin_amdgcn_sdot8(int(t[r][j]), int(xw[b][4 * l + j]), d[r][b], false);
    }
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) pr[r][b] = float(d[r][b]);
  } else if constexpr (BITS == 8) {
    // codes as signed bytes q - 128 against the byte limb words; the limb
    // sums combine in fp32
    int d[G][NB][3];
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) d[r][b][0] = d[r][b][1] = d[r][b][2] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int l = 0; l < 3; ++l)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int r = 0; r < G; ++r)
            d[r][b][l] = __builtin_amdgcn_sdot4(int(wc[r][i] ^ 0x80808080u), int(xw[b][8 * l + i]),
                                                d[r][b][l], false);
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        pr[r][b] = float(d[r][b][0]) + 256.f * float(d[r][b][1]) + 65536.f * float(d[r][b][2]);
  } else {
    // 3-bit codes: bit-field extracts, conversions, fp32 fused multiply-adds
    float acc[G][NB];
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
#pragma unroll
    for (int k = 0; k < CODES; ++k) {
      const int bit = 3 * k, i = bit >> 5, sh = bit & 31;
      float q[G];
#pragma unroll
      for (int r = 0; r < G; ++r) {
        uint32_t v = wc[r][i] >> sh;
        if (sh + 3 > 32) v |= wc[r][i + 1] << (32 - sh);
        q[r] = float(v & 7u);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float xk = __uint_as_float(xw[b][k]);
#pragma unroll
        for (int r = 0; r < G; ++r) acc[r][b] = __builtin_fmaf(q[r], xk, acc[r][b]);
      }
    }
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) pr[r][b] = acc[r][b];
  }
}

// v[r * NB + b] for the group's rows: with one grid per row the unscaled
// chunk product unit * sum_k q m (the grid applies to the row's total); with
// groups of 128 columns scale unit (sum_k q m - zero sum_k m) for the chunk's
// group (fp32 products: unit = 1, m = x).
template <int BITS, int NB, bool GROUPED>
__device__ inline void group_values(const uint32_t (&wc)[G][BITS], const float* scg,
                                    const float* zrg, int ngroups, int64_t g, bool act, int last,
                                    const uint32_t (&xw)[NB][XW], const float (&cs)[NB],
                                    float (&v)[G * NB]) {
  constexpr bool INT = BITS != 3;
  float prg[G][NB];
  group_dot<BITS, NB>(wc, xw, prg);
#pragma unroll
  for (int r = 0; r < G; ++r) {
    const float(&pr)[NB] = prg[r];
    if constexpr (GROUPED) {
      const int rr = min(r, last);
      const float sc = act ? scg[rr * ngroups + g] : 0.f;
      float zr = act ? zrg[rr * ngroups + g] : 0.f;
      zr -= code_offset(BITS);  // the products used q - offset
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float u = INT ? sc * __uint_as_float(xw[b][W_UNIT]) : sc;
        v[r * NB + b] = u * (pr[b] - zr * cs[b]);
      }
    } else {
#pragma unroll
      for (int b = 0; b < NB; ++b) v[r * NB + b] = INT ? __uint_as_float(xw[b][W_UNIT]) * pr[b] : pr[b];
    }
  }
}

// Waves per workgroup of the product: 16 where the kernel fits 128 VGPRs
// (one vector, 2-bit codes, one grid per row), else 8 (256 VGPRs).
constexpr int max_waves(int bits, int nb, bool grouped) {
  return nb == 1 && bits == 2 && !grouped ? 16 : 8;
}

// y1[b0 + b][rows] = W^'[rows] x2[b0 + b] for b < nb (nb <= NB), rows
// blockIdx.x * rpw .. + rpw - 1 (rpw a multiple of G, rpw * NB <= SLOT).
// Wave w of the workgroup takes K tiles w, w + waves, ...
template <int BITS, int NB, bool GROUPED>
__global__ __launch_bounds__(64 * max_waves(BITS, NB, GROUPED)) void qmatvec_kernel(
    const uint32_t* __restrict__ packed, int rw, const float* __restrict__ scale,
    const float* __restrict__ zero, int ngroups, const uint32_t* __restrict__ xq, int64_t nchunk,
    int64_t d_out, int nkt, int rpw, int b0, int nb, float* __restrict__ y1) {
  constexpr bool INT = BITS != 3;
  constexpr int NV = G * NB;          // values per group
  constexpr int LGV = NV == 8 ? 3 : NV == 16 ? 4 : 5;
  __shared__ float red[max_waves(BITS, NB, GROUPED)][SLOT];
  __shared__ float redx[max_waves(BITS, NB, GROUPED)][4];  // sum of x2, one grid per row
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int64_t rbeg = int64_t(blockIdx.x) * rpw;
  const int nrows = int(min(int64_t(rpw), d_out - rbeg));
  for (int i = lane; i < SLOT; i += LANES) red[w][i] = 0.f;  // this wave's slots only
  if (lane < 4) redx[w][lane] = 0.f;
  // after the butterfly lane L holds value L >> (6 - LGV) = row * NB + vector
  const int vi = lane >> (6 - LGV), vr = vi / NB, vb = vi % NB;

  // The wave's work: K tiles w, w + nw, ... times the row groups, in that
  // order. The codes of step it + 1 are loaded while step it is computed.
  const int ngrp = (nrows + G - 1) / G;
  const int steps = ((nkt - 1 - w) / nw + 1) * ngrp;
  auto step_kt = [&](int it) { return w + (it / ngrp) * nw; };
  auto step_gi = [&](int it) { return (it % ngrp) * G; };
  auto issue = [&](int it, uint32_t (&dst)[G][BITS]) {
    const int64_t c = min(int64_t(step_kt(it)) * LANES + lane, nchunk - 1);
    const int gi = step_gi(it);
    load_group<BITS, G>(packed + c * BITS + (rbeg + gi) * rw, rw, min(G, nrows - gi) - 1, dst);
  };
  // the next step's codes load during this step where the registers allow
  constexpr bool PREFETCH = G * BITS <= 32 || (NB == 1 && G * BITS <= 64);
  uint32_t xw[NB][XW];
  float cs[NB];
  int cur_kt = -1;
  uint32_t wn[PREFETCH ? G : 1][BITS];
  for (int it = 0; it < steps; ++it) {
    const int kt = step_kt(it), gi = step_gi(it);
    const int64_t c = int64_t(kt) * LANES + lane;
    const bool act = c < nchunk;
    if (kt != cur_kt) {
      // a new K tile: this lane's chunk of the prepared input, loaded
      // ahead of the step's codes
      cur_kt = kt;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int bb = b < nb ? b0 + b : b0;  // unused slots repeat a valid vector
        const uint4* p = reinterpret_cast<const uint4*>(xq + (bb * nchunk + min(c, nchunk - 1)) * XW);
        constexpr int NQ = INT ? 7 : 8;  // integer chunks: words 0 .. 27
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint4 u = q < NQ ? p[q] : make_uint4(0u, 0u, 0u, 0u);
          xw[b][4 * q] = act ? u.x : 0u;
          xw[b][4 * q + 1] = act ? u.y : 0u;
          xw[b][4 * q + 2] = act ? u.z : 0u;
          xw[b][4 * q + 3] = act ? u.w : 0u;
        }
      }
      if constexpr (PREFETCH) {
        if (it == 0) issue(0, wn);
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        if constexpr (INT) {
          cs[b] = __uint_as_float(xw[b][W_MSUM]);
        } else {
          float sum = 0.f;
#pragma unroll
          for (int k = 0; k < CODES; k += 2)
            sum += __uint_as_float(xw[b][k]) + __uint_as_float(xw[b][k + 1]);
          cs[b] = sum;
        }
      }
      if constexpr (!GROUPED) {
        // the zero-point term of a row-wide grid needs sum_j x2_j
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float t = INT ? __uint_as_float(xw[b][W_UNIT]) * cs[b] : cs[b];
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
          if (lane == 0) redx[w][b] += t;
        }
      }
    }
    uint32_t wc[G][BITS];
    if constexpr (PREFETCH) {
#pragma unroll
      for (int r = 0; r < G; ++r)
#pragma unroll
        for (int i = 0; i < BITS; ++i) wc[r][i] = wn[r][i];
      if (it + 1 < steps) issue(it + 1, wn);
    } else {
      issue(it, wc);
    }
    const int last = min(G, nrows - gi) - 1;
    const int64_t r0 = rbeg + gi;
    const int64_t g = GROUPED ? c / (128 / CODES) : 0;
    float v[NV];
    group_values<BITS, NB, GROUPED>(wc, scale + r0 * ngroups, zero + r0 * ngroups, ngroups, g, act,
                                    last, xw, cs, v);
    const float tot = fold_all<NV>(v, lane);
    if ((lane & ((64 >> LGV) - 1)) == 0 && gi + vr < nrows) red[w][(gi + vr) * NB + vb] += tot;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nrows * NB; i += blockDim.x) {
    const int r = i / NB, b = i % NB;
    if (b < nb) {
      float s = 0.f;
      for (int u = 0; u < nw; ++u) s += red[u][i];
      if constexpr (!GROUPED) {
        float xs = 0.f;
        for (int u = 0; u < nw; ++u) xs += redx[u][b];
        const int64_t row = rbeg + r;
        const float zr = zero[row] - code_offset(BITS);  // the products used q - offset
        s = scale[row] * (s - zr * xs);
      }
      y1[(b0 + b) * d_out + rbeg + r] = s;
    }
  }
}

template <int BITS, int NB>
void launch_qmatvec_nb(const uint32_t* packed, int64_t rw, const float* scale, const float* zero,
                       int ngroups, bool grouped, const uint32_t* xq, int64_t nchunk, int64_t d_out,
                       int b0, int nb, float* y1, hipStream_t s) {
  const int nkt = int(cdiv(nchunk, LANES));
  const int nw = std::min(nkt, max_waves(BITS, NB, grouped));
  // rows per workgroup: the most (up to SLOT / NB) that leave >= 256
  // workgroups, one per compute unit
  int rpw = SLOT / NB;
  while (rpw > G && cdiv(d_out, rpw) < 256) rpw >>= 1;
  const unsigned blocks = unsigned(cdiv(d_out, rpw));
  if (grouped)
    qmatvec_kernel<BITS, NB, true><<<blocks, 64 * nw, 0, s>>>(packed, int(rw), scale, zero, ngroups, xq,
                                                             nchunk, d_out, nkt, rpw, b0, nb, y1);
  else
    qmatvec_kernel<BITS, NB, false><<<blocks, 64 * nw, 0, s>>>(packed, int(rw), scale, zero, ngroups, xq,
                                                              nchunk, d_out, nkt, rpw, b0, nb, y1);
}

template <int BITS>
kq_status run_bits(const uint32_t* packed, int64_t rw, const float* scale, const float* zero,
                   int ngroups, bool grouped, const float* s_x, const int8_t* si, int64_t bi,
                   const float* x, int64_t batch, int64_t d_out, int64_t d_in, uint32_t* xq,
                   float* y1, hipStream_t s) {
  const int64_t Li = transform_len(d_in, bi);
  const unsigned tin = unsigned(std::max<int64_t>(64, std::min<int64_t>(1024, Li / 4)));
  with_lgb(ilog2(bi), [&](auto C) {
    transform_in_kernel<BITS, decltype(C)::value><<<unsigned(batch * (d_in / Li)), tin, 0, s>>>(
        x, d_in, ilog2(Li), ilog2(bi), si, s_x, float(1.0 / std::sqrt(double(bi))), xq);
  });
  KQ_HIP(hipGetLastError());
  const int64_t nchunk = d_in / CODES;
  KQ_TRY(mark_kernel(KQ_OP_APPLY_QUANTIZED, 0, s));
  for (int64_t b0 = 0; b0 < batch; b0 += 4) {
    const int nb = int(std::min<int64_t>(4, batch - b0));
    if (nb == 1)
      launch_qmatvec_nb<BITS, 1>(packed, rw, scale, zero, ngroups, grouped, xq, nchunk, d_out, int(b0), 1, y1, s);
    else if (nb == 2)
      launch_qmatvec_nb<BITS, 2>(packed, rw, scale, zero, ngroups, grouped, xq, nchunk, d_out, int(b0), 2, y1, s);
    else
      launch_qmatvec_nb<BITS, 4>(packed, rw, scale, zero, ngroups, grouped, xq, nchunk, d_out, int(b0), nb, y1, s);
    KQ_HIP(hipGetLastError());
  }
  return mark_kernel(KQ_OP_APPLY_QUANTIZED, 1, s);
}


// ---------------------------------------------------------------------------
// Matrix-core path for 2-bit codes with one grid per row (d_in a multiple of
// 512): v_mfma_scale_f32_16x16x128_f8f6f4, A = codes as fp4 (e2m1), B = the
// transformed input as fp8 (e4m3) digits with E8M0 block scales.
//
// Operand layout of the instruction (16 x 16 x 128; lane l, G = l / 16):
//   A: row l % 16, K 32 G + j in nibble j of its first four registers;
//   B: column l % 16, K 16 G + (j % 16) + 64 (j / 16) in byte j;
//   scale byte of lane l (selected by op_sel): K block G (32 values) of its
//   row (A) or column (B); C: lane l holds rows 4 G + i, column l % 16.
// The e2m1 encodings 0-3 are the values 0, 0.5, 1, 1.5: a 2-bit code q is
// the fp4 value q / 2 as it stands, so the decode is two nibble masks per
// packed word (0x33333333 after shifts of 0 and 2).
// Codes: over a super-step of 512 columns a lane (row r, G) reads codes
// 64 G .. 64 G + 63 and 256 + 64 G .. 256 + 64 G + 63 (two 16-byte loads;
// each load instruction covers 64 contiguous bytes of 16 rows), and step
// q = 2 h + o takes the 32 codes from 256 h + 64 G + 32 o; nibble j holds
// code p(j) = 2 i + (j / 8 odd) + 16 (j >= 16) of them, i = j % 8.
// Input: each 32-value chunk in fixed point against its own exponent e
// (m = rint(x 2^(22 - e)), as in the integer path), m = sum_l n_l 16^l with
// six digits n_l in [-8, 7], exact in e4m3. Column n = 6 v + l of B holds
// digit l of vector v; its block scale is 2^(4 l + e - 21) (the 2 undoes the
// halved codes). The instruction's sum is then sum_k q_k x_k, to fp32
// accumulation (measured error <= 2^-23 of the sum of |terms|).
constexpr int MX_SS = 512;         // columns per super-step
constexpr int MX_DIG = 6;          // digits per value
constexpr int MX_BYTES = 4 * 4 * MX_DIG * 32;  // digit bytes per super-step and vector
constexpr int MX_SCALES = 4 * MX_DIG;          // scale words per super-step and vector

// e4m3 encoding of an integer n in [-16, 16] (exact: 3 mantissa bits), by
// the hardware conversion
__device__ inline uint8_t e4m3_int(int n) {
  return uint8_t(__builtin_amdgcn_cvt_pk_fp8_f32(float(n), 0.f, 0, false) & 0xFF);
}

// x2 = gain * H_blk (x[b] sign_in / s_x) over L columns, written as B digits
// xb[b][S][q][g][l][32 bytes], scale words xs[b][S][G][l] (byte q) and the
// chunk's sum of x2 in xsum[b][blockIdx % per_row].
template <int LGB>
__global__ __launch_bounds__(1024) void transform_in_mx_kernel(
    const float* __restrict__ x, int64_t d_in, int lgL, int lgb, const int8_t* __restrict__ si,
    const float* __restrict__ s_x, float gain, uint8_t* __restrict__ xb, uint32_t* __restrict__ xs,
    float* __restrict__ xsum) {
  __shared__ float s[TCHP];
  __shared__ __align__(16) uint8_t dig[TCH * MX_DIG];  // digit bytes in output order
  __shared__ uint32_t scl[TCH / 32 * MX_DIG];
  __shared__ float part[32];
  const int L = 1 << lgL;
  const int64_t per_row = d_in >> lgL;
  const int64_t b = blockIdx.x / per_row;
  const int64_t c0 = int64_t(blockIdx.x % per_row) << lgL;
  const float* src = x + b * d_in + c0;
  for (int e = 4 * threadIdx.x; e < L; e += 4 * blockDim.x) {
    const float4 v = *reinterpret_cast<const float4*>(src + e);
    const float4 sx = *reinterpret_cast<const float4*>(s_x + c0 + e);
    s[padi(e)] = v.x * float(si[c0 + e]) / sx.x;
    s[padi(e + 1)] = v.y * float(si[c0 + e + 1]) / sx.y;
    s[padi(e + 2)] = v.z * float(si[c0 + e + 2]) / sx.z;
    s[padi(e + 3)] = v.w * float(si[c0 + e + 3]) / sx.w;
  }
  for (int i = threadIdx.x; i < L / 32 * MX_DIG; i += blockDim.x) scl[i] = 0u;
  __syncthreads();
  lds_fwht_blk<LGB>(s, L, lgb);
  float tsum = 0.f;
  // one value per lane; the 32 lanes of a half-wave hold one chunk
  for (int e = threadIdx.x; e < L; e += blockDim.x) {
    const float v = gain * s[padi(e)];
    tsum += v;
    float mx = fabsf(v);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    int ex = 0;
    if (mx > 0.f) frexpf(mx, &ex);  // mx = f 2^ex, 1/2 <= f < 1
    // chunks whose smallest digit scale would fall below E8M0's range hold
    // values under 2^-148: taken as zero
    const bool keep = mx > 0.f && ex - 21 >= -127;
    const int m = keep ? int(rintf(ldexpf(v, 22 - ex))) : 0;
    // position of this code in the operand layout
    const int u = e & (MX_SS - 1), S = e / MX_SS;
    const int G = (u >> 6) & 3, q = 2 * (u >> 8) + ((u >> 5) & 1), p = u & 31;
    const int j = 8 * (2 * (p >> 4) + (p & 1)) + ((p & 15) >> 1);
    const int k = 32 * G + j;
    const int g = (k & 63) >> 4, jb = (k & 15) + 16 * (k >> 6);
    int r = m;
#pragma unroll
    for (int l = 0; l < MX_DIG; ++l) {
      const int n = ((r + 8) & 15) - 8;  // balanced base-16 digit
      r = (r - n) >> 4;
      dig[(((S * 4 + q) * 4 + g) * MX_DIG + l) * 32 + jb] = e4m3_int(n);
    }
    if ((e & 31) == 0) {
#pragma unroll
      for (int l = 0; l < MX_DIG; ++l) {
        const uint32_t sc = keep ? uint32_t(127 + 4 * l + ex - 21) : 0u;
        atomicOr(&scl[(S * 4 + G) * MX_DIG + l], sc << (8 * q));
      }
    }
  }
  // workgroup sum of x2 (fixed order: lanes, then waves)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tsum += __shfl_xor(tsum, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = tsum;
  __syncthreads();
  const int64_t nss = d_in / MX_SS, S0 = c0 / MX_SS;
  uint8_t* dstb = xb + (b * nss + S0) * MX_BYTES;
  for (int i = 16 * threadIdx.x; i < L / MX_SS * MX_BYTES; i += 16 * blockDim.x)
    *reinterpret_cast<uint4*>(dstb + i) = *reinterpret_cast<const uint4*>(dig + i);
  uint32_t* dsts = xs + (b * nss + S0) * MX_SCALES;
  for (int i = threadIdx.x; i < L / MX_SS * MX_SCALES; i += blockDim.x) dsts[i] = scl[i];
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < int(blockDim.x >> 6); ++w) t += part[w];
    xsum[b * per_row + blockIdx.x % per_row] = t;
  }
}

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane from global memory straight into LDS: lane i's land at
// lds_addr + 16 i. Complete once vmcnt has counted the load down.
__device__ inline void a4_dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory", "m0");
}

template <int N>
__device__ inline void a4_wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Sum over the 16 lanes of a DPP row, left in every lane of the row: lane
// pairs (quad_perm 1 0 3 2), then quads (2 3 0 1), then the mirrored half
// row adds the other quad of its 8 lanes and the mirrored row the other 8.
__device__ inline float row16_sum(float t) {
  t += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(t), 0xB1, 0xF, 0xF, false));
  t += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(t), 0x4E, 0xF, 0xF, false));
  t += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(t), 0x141, 0xF, 0xF, false));
  t += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(t), 0x140, 0xF, 0xF, false));
  return t;
}

// An empty use of a wave's B operands, ordered with the DMA asm around it.
__device__ inline void mx_hold_b(const v8i_t (&b)[4], uint32_t sc) {
  asm volatile("" : : "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]), "v"(sc));
}

// Partial products of the matrix-core path. Workgroup (row block rb, K
// group g) covers rows rb * rpw .. + rpw - 1 and super-steps g * nw .. +
// nw - 1, one per wave: y1p[g][b0 + v][row] = scale (sum over those
// columns of W^' x2, less zero sum x2 in group 0) for v < NV, so the K
// groups' planes add up to y1. A 16-column B tile holds the digit columns of
// two vectors; NV > 2 takes a second tile, which shares every decoded A
// operand. A wave loads its super-step's B operands once and streams its
// 16-row code tiles through a private LDS ring of `depth` stages (one
// 16-row tile, 2 KB, per stage), filled by DMA `depth - 1` tiles ahead.
constexpr int MX_STAGE = 2048;
template <int NV>
__global__ __launch_bounds__(1024) void qmatvec_mx_kernel(
    const uint32_t* __restrict__ packed, int rw, const float* __restrict__ scale,
    const float* __restrict__ zero, const uint8_t* __restrict__ xb, const uint32_t* __restrict__ xs,
    const float* __restrict__ xsum, int nparts, int64_t nss, int64_t d_out, int kgroups, int rpw,
    int depth, int b0, int64_t batch, float* __restrict__ y1p) {
  constexpr int NT = (NV + 1) / 2;  // B tiles
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int g = blockIdx.x % kgroups;
  const int64_t rbeg = int64_t(blockIdx.x / kgroups) * rpw;
  const int nrows = int(min(int64_t(rpw), d_out - rbeg));
  const int64_t S = int64_t(g) * nw + w;  // this wave's super-step, < nss
  float* red = reinterpret_cast<float*>(lds + size_t(nw) * depth * MX_STAGE);  // [nw][rpw][NV]
  const uint32_t ring = uint32_t(reinterpret_cast<uintptr_t>(lds)) + uint32_t(w * depth * MX_STAGE);
  const int n = lane & 15, G = lane >> 4;
  const int lcol = n % MX_DIG;
  // tile tt, column n: digit lcol of vector 2 tt + n / 6; columns past the
  // vectors' digits stay zero
  bool bcol[NT];
  int vcol[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    bcol[tt] = n < MX_DIG * min(2, NV - 2 * tt);
    vcol[tt] = bcol[tt] ? 2 * tt + n / MX_DIG : 0;
  }
  // B operands first: they are in flight before any DMA
  v8i_t bop[NT][4];
  uint32_t bsc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const uint8_t* bp = xb + ((b0 + vcol[tt]) * nss + S) * MX_BYTES;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4* p = reinterpret_cast<const uint4*>(bp + ((q * 4 + G) * MX_DIG + lcol) * 32);
      const uint4 lo = bcol[tt] ? p[0] : make_uint4(0u, 0u, 0u, 0u);
      const uint4 hi = bcol[tt] ? p[1] : make_uint4(0u, 0u, 0u, 0u);
      bop[tt][q] = v8i_t{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
    }
    bsc[tt] = bcol[tt] ? xs[((b0 + vcol[tt]) * nss + S) * MX_SCALES + G * MX_DIG + lcol] : 0u;
  }
  // tile t of the codes: rows rbeg + 16 t + n (past the end: the last row,
  // not stored), this lane's 16 bytes of each 64-byte half of the super-step
  const int items = (nrows + 15) / 16;
  const uint8_t* arow = reinterpret_cast<const uint8_t*>(packed + S * (MX_SS / 16) + G * 4);
  auto issue = [&](int t) {
    const int64_t row = rbeg + min(16 * t + n, nrows - 1);
    const uint8_t* src = arow + row * int64_t(rw) * 4;
    const uint32_t dst = ring + uint32_t((t % depth) * MX_STAGE);
    a4_dma16(src, dst);
    a4_dma16(src + 64, dst + 1024);
  };
  issue(0);
  a4_wait_vm<0>();  // B and tile 0
  // B is used here, so the compiler's own wait for it falls at this point,
  // before any later DMA is in flight
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) mx_hold_b(bop[tt], bsc[tt]);
  int issued = 1;
  for (int it = 0; it < items; ++it) {
    if (it > 0) {
      // tile it done; the tiles after it may stay in flight (two DMAs each)
      switch (issued - it - 1) {
        case 0: a4_wait_vm<0>(); break;
        case 1: a4_wait_vm<2>(); break;
        case 2: a4_wait_vm<4>(); break;
        case 3: a4_wait_vm<6>(); break;
        case 4: a4_wait_vm<8>(); break;
        case 5: a4_wait_vm<10>(); break;
        case 6: a4_wait_vm<12>(); break;
        default: a4_wait_vm<14>(); break;
      }
    }
    // refill: the slot of tile it - 1 is free, its reads are done
    while (issued < items && issued < it + depth) issue(issued++);
    const uint8_t* st = lds + size_t(w * depth + it % depth) * MX_STAGE;
    const uint4 lo = *reinterpret_cast<const uint4*>(st + lane * 16);
    const uint4 hi = *reinterpret_cast<const uint4*>(st + 1024 + lane * 16);
    const uint32_t wd[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    v4f_t acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = v4f_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t x0 = wd[2 * q], x1 = wd[2 * q + 1];
      const v8i_t aop = {int(x0 & 0x33333333u), int((x0 >> 2) & 0x33333333u),
                         int(x1 & 0x33333333u), int((x1 >> 2) & 0x33333333u), 0, 0, 0, 0};
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const int sc = int(bsc[tt]);
        if (q == 0) acc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[tt][0], acc[tt], 4, 0, 0, 0x7f7f7f7f, 0, sc);
        if (q == 1) acc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[tt][1], acc[tt], 4, 0, 0, 0x7f7f7f7f, 1, sc);
        if (q == 2) acc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[tt][2], acc[tt], 4, 0, 0, 0x7f7f7f7f, 2, sc);
        if (q == 3) acc[tt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[tt][3], acc[tt], 4, 0, 0, 0x7f7f7f7f, 3, sc);
      }
    }
    // acc[tt][i] = C[4 G + i][n] of B tile tt: add the digit columns of each vector
#pragma unroll
    for (int v = 0; v < NV; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = v / 2;
        const float t = row16_sum((bcol[tt] && vcol[tt] == v) ? acc[tt][i] : 0.f);
        const int r = 16 * it + 4 * G + i;
        if (n == 0 && r < nrows) red[(w * rpw + r) * NV + v] = t;
      }
  }
  __syncthreads();
  float* dst = y1p + int64_t(g) * batch * d_out;
  for (int i = threadIdx.x; i < nrows * NV; i += blockDim.x) {
    const int r = i / NV, v = i % NV;
    float acc = 0.f;
    for (int u = 0; u < nw; ++u) acc += red[u * rpw * NV + i];
    const int64_t row = rbeg + r;
    if (g == 0) {
      float xs_sum = 0.f;
      for (int pp = 0; pp < nparts; ++pp) xs_sum += xsum[(b0 + v) * nparts + pp];
      acc -= zero[row] * xs_sum;
    }
    dst[(b0 + v) * d_out + row] = scale[row] * acc;
  }
}

// Launch shape of the matrix-core product: K groups of at most 16
// super-steps (one per wave), then rows per workgroup (16 .. 128) as many
// as still leave >= 256 workgroups, then the ring depth that the LDS holds.
struct MxPlan {
  int kgroups, nw, rpw;
};
MxPlan mx_plan(int64_t d_out, int64_t d_in) {
  const int64_t nss = d_in / MX_SS;
  int64_t kg = 1;
  while (nss % kg || nss / kg > 16) ++kg;
  int rpw = 128;
  while (rpw > 16 && cdiv(d_out, rpw) * kg < 256) rpw >>= 1;
  return MxPlan{int(kg), int(nss / kg), rpw};
}
int64_t mx_planes(int64_t d_in) { return d_in % MX_SS == 0 ? mx_plan(16, d_in).kgroups : 1; }

constexpr size_t MX_LDS = 160 * 1024;
template <int NV>
kq_status launch_qmatvec_mx(const uint32_t* packed, int64_t rw, const float* scale, const float* zero,
                            const uint8_t* xb, const uint32_t* xs, const float* xsum, int nparts,
                            int64_t nss, int64_t d_out, int b0, int64_t batch, float* y1p, hipStream_t s) {
  const MxPlan pl = mx_plan(d_out, nss * MX_SS);
  const size_t red_bytes = size_t(pl.nw) * pl.rpw * NV * sizeof(float);
  const int ntile = pl.rpw / 16;
  const int fit = int((MX_LDS - red_bytes) / (size_t(pl.nw) * MX_STAGE));
  const int depth = std::max(1, std::min({8, ntile, fit}));
  const size_t bytes = size_t(pl.nw) * depth * MX_STAGE + red_bytes;
  KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(qmatvec_mx_kernel<NV>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(bytes)));
  qmatvec_mx_kernel<NV><<<unsigned(cdiv(d_out, pl.rpw) * pl.kgroups), 64 * pl.nw, bytes, s>>>(
      packed, int(rw), scale, zero, xb, xs, xsum, nparts, nss, d_out, pl.kgroups, pl.rpw, depth, b0,
      batch, y1p);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

kq_status run_mx(const uint32_t* packed, int64_t rw, const float* scale, const float* zero,
                 const float* s_x, const int8_t* si, int64_t bi, const float* x, int64_t batch,
                 int64_t d_out, int64_t d_in, uint8_t* xb, uint32_t* xs, float* xsum, float* y1,
                 hipStream_t s) {
  const int64_t Li = transform_len(d_in, bi);
  const int64_t nss = d_in / MX_SS, nparts = d_in / Li;
  with_lgb(ilog2(bi), [&](auto C) {
    transform_in_mx_kernel<decltype(C)::value>
        <<<unsigned(batch * nparts), unsigned(std::min<int64_t>(1024, Li / 4)), 0, s>>>(
            x, d_in, ilog2(Li), ilog2(bi), si, s_x, float(1.0 / std::sqrt(double(bi))), xb, xs, xsum);
  });
  KQ_HIP(hipGetLastError());
  KQ_TRY(mark_kernel(KQ_OP_APPLY_QUANTIZED, 0, s));
  for (int64_t b0 = 0; b0 < batch; b0 += 4) {
    const int64_t left = batch - b0;
    const int b = int(b0);
    if (left >= 4)
      KQ_TRY(launch_qmatvec_mx<4>(packed, rw, scale, zero, xb, xs, xsum, int(nparts), nss, d_out, b, batch, y1, s));
    else if (left == 3)
      KQ_TRY(launch_qmatvec_mx<3>(packed, rw, scale, zero, xb, xs, xsum, int(nparts), nss, d_out, b, batch, y1, s));
    else if (left == 2)
      KQ_TRY(launch_qmatvec_mx<2>(packed, rw, scale, zero, xb, xs, xsum, int(nparts), nss, d_out, b, batch, y1, s));
    else
      KQ_TRY(launch_qmatvec_mx<1>(packed, rw, scale, zero, xb, xs, xsum, int(nparts), nss, d_out, b, batch, y1, s));
  }
  return mark_kernel(KQ_OP_APPLY_QUANTIZED, 1, s);
}


// ---- Weights and activations both quantized: 2-bit codes, 4-bit inputs.
// Each vector's rotated input x2 = V S_X^-1 x is rounded on a symmetric grid
// of its own: s = (clip max_k |x2_k|) / 7 and a_k = clamp(rint(x2_k / s), -8,
// 7), in fp32 with ties to even (an all-zero vector has s = 0, a = 0). The
// product is then integer arithmetic on the matrix cores: the codes enter
// as fp4 (q / 2) as in the path above and the input codes as e4m3 integers
// with block scale 2, sixteen vectors in the 16 B columns of one
// v_mfma_scale_f32_16x16x128_f8f6f4. Every partial sum sum_k q_k a_k is an
// integer below 3 * 8 * d_in < 2^24, so fp32 holds it exactly and the
// order of the sums does not matter; y1 = scale s (sum q a - zero sum a).
//
// B layout: vector tile T (16 vectors), super-step S (512 columns), step q,
// lane l = 16 g + n: 32 bytes at xa[((T nss + S) 4 + q) 64 + l] for vector
// 16 T + n; column u of the super-step sits at (q, g, byte) as in the MX
// placement above. Staged per vector as (q 4 + g) 32 + byte.
constexpr int A4_TILE = 16;           // vectors per column tile
constexpr int A4_SSB = 4 * 64 * 32;   // bytes per tile and super-step
constexpr float A4_QMAX = 7.f;

__device__ inline int a4_slot(int u) {
  const int G = (u >> 6) & 3, q = 2 * (u >> 8) + ((u >> 5) & 1), p = u & 31;
  const int j = 8 * (2 * (p >> 4) + (p & 1)) + ((p & 15) >> 1);
  const int k = 32 * G + j;
  const int g = (k & 63) >> 4, jb = (k & 15) + 16 * (k >> 6);
  return (q * 4 + g) * 32 + jb;
}

__device__ inline int a4_code(float v, float s) {
  if (!(s > 0.f)) return 0;
  return int(fminf(fmaxf(rintf(v / s), -8.f), A4_QMAX));
}

// Largest value over the workgroup (every thread gets it). part: >= 16 floats.
__device__ inline float block_max(float m, float* part) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = 0.f;
  for (int w = 0; w < int(blockDim.x >> 6); ++w) r = fmaxf(r, part[w]);
  return r;
}

// Quantize columns e .. e + 3 of a super-step-aligned run of one vector
// (values v) into the staging bytes and, if wanted, the caller's codes.
__device__ inline int a4_put4(float4 v, float s, int e, uint8_t* stg, int8_t* codes_out) {
  const int c0 = a4_code(v.x, s), c1 = a4_code(v.y, s), c2 = a4_code(v.z, s), c3 = a4_code(v.w, s);
  const int base = e & ~(MX_SS - 1), u = e & (MX_SS - 1);
  stg[base + a4_slot(u)] = e4m3_int(c0);
  stg[base + a4_slot(u + 1)] = e4m3_int(c1);
  stg[base + a4_slot(u + 2)] = e4m3_int(c2);
  stg[base + a4_slot(u + 3)] = e4m3_int(c3);
  if (codes_out)
    *reinterpret_cast<char4*>(codes_out + e) = make_char4(char(c0), char(c1), char(c2), char(c3));
  return c0 + c1 + c2 + c3;
}

// Staged bytes of super-steps [S0, S0 + nS) of vector b -> their places in xa.
__device__ inline void a4_store(const uint8_t* stg, int nS, int64_t b, int64_t S0, int64_t nss,
                                uint8_t* __restrict__ xa) {
  const int64_t T = b / A4_TILE, n = b % A4_TILE;
  for (int i = threadIdx.x; i < nS * 32; i += blockDim.x) {
    const int S = i >> 5, r = (i >> 1) & 15, h = i & 1;  // run r = 4 q + g, half h
    const int q = r >> 2, g = r & 3;
    uint8_t* dst = xa + ((T * nss + S0 + S) * 4 + q) * (64 * 32) + (16 * g + n) * 32 + 16 * h;
    *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(stg + S * MX_SS + r * 32 + 16 * h);
  }
}

// x2 = gain * H_blk (x[b] sign_in / s_x) over L columns. FUSED (the chunk is
// the whole vector): quantize it here, with the vector's code sum in
// asum[b]. Otherwise write x2 and the chunk's largest magnitude for
// quantize_a4_kernel.
template <bool FUSED, int LGB>
__global__ __launch_bounds__(1024) void transform_in_a4_kernel(
    const float* __restrict__ x, int64_t d_in, int lgL, int lgb, const int8_t* __restrict__ si,
    const float* __restrict__ s_x, float gain, float clip, float* __restrict__ x2,
    float* __restrict__ pmax, uint8_t* __restrict__ xa, float* __restrict__ ascale,
    int* __restrict__ asum, int8_t* __restrict__ codes_out, float* __restrict__ scale_out) {
  __shared__ float s[TCHP];
  __shared__ __align__(16) uint8_t stg[FUSED ? TCH : 16];
  __shared__ float part[16];
  __shared__ int ipart[16];
  const int L = 1 << lgL;
  const int64_t per_row = d_in >> lgL;
  const int64_t b = blockIdx.x / per_row;
  const int64_t c0 = int64_t(blockIdx.x % per_row) << lgL;
  const float* src = x + b * d_in + c0;
  for (int e = 4 * threadIdx.x; e < L; e += 4 * blockDim.x) {
    const float4 v = *reinterpret_cast<const float4*>(src + e);
    const float4 sx = *reinterpret_cast<const float4*>(s_x + c0 + e);
    s[padi(e)] = v.x * float(si[c0 + e]) / sx.x;
    s[padi(e + 1)] = v.y * float(si[c0 + e + 1]) / sx.y;
    s[padi(e + 2)] = v.z * float(si[c0 + e + 2]) / sx.z;
    s[padi(e + 3)] = v.w * float(si[c0 + e + 3]) / sx.w;
  }
  __syncthreads();
  lds_fwht_blk<LGB>(s, L, lgb);
  __syncthreads();
  float mx = 0.f;
  for (int e = 4 * threadIdx.x; e < L; e += 4 * blockDim.x) {
    const float4 v = make_float4(gain * s[padi(e)], gain * s[padi(e + 1)], gain * s[padi(e + 2)],
                                 gain * s[padi(e + 3)]);
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    if (!FUSED) *reinterpret_cast<float4*>(x2 + b * d_in + c0 + e) = v;
  }
  mx = block_max(mx, part);
  if constexpr (!FUSED) {
    if (threadIdx.x == 0) pmax[blockIdx.x] = mx;
  } else {
    const float sc = (clip * mx) / A4_QMAX;
    int8_t* co = codes_out ? codes_out + b * d_in : nullptr;
    int cs = 0;
    for (int e = 4 * threadIdx.x; e < L; e += 4 * blockDim.x) {
      const float4 v = make_float4(gain * s[padi(e)], gain * s[padi(e + 1)], gain * s[padi(e + 2)],
                                   gain * s[padi(e + 3)]);
      cs += a4_put4(v, sc, e, stg, co);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cs += __shfl_xor(cs, o);
    if ((threadIdx.x & 63) == 0) ipart[threadIdx.x >> 6] = cs;
    __syncthreads();
    a4_store(stg, L / MX_SS, b, 0, d_in / MX_SS, xa);
    if (threadIdx.x == 0) {
      int t = 0;
      for (int w = 0; w < int(blockDim.x >> 6); ++w) t += ipart[w];
      asum[b] = t;
      ascale[b] = sc;
      if (scale_out) scale_out[b] = sc;
    }
  }
}

// One workgroup of 128 threads per (vector, super-step): the vector's scale
// from its chunk maxima, then its 512 values quantized and placed; the sum
// of their codes goes to asum[b][S].
__global__ __launch_bounds__(128) void quantize_a4_kernel(
    const float* __restrict__ x2, const float* __restrict__ pmax, int nparts, int64_t d_in,
    int64_t nss, float clip, uint8_t* __restrict__ xa, float* __restrict__ ascale,
    int* __restrict__ asum, int8_t* __restrict__ codes_out, float* __restrict__ scale_out) {
  __shared__ __align__(16) uint8_t stg[MX_SS];
  __shared__ int ipart[2];
  const int64_t b = blockIdx.x / nss, S = blockIdx.x % nss;
  float mx = 0.f;
  for (int p = 0; p < nparts; ++p) mx = fmaxf(mx, pmax[b * nparts + p]);
  const float sc = (clip * mx) / A4_QMAX;
  const int e = 4 * threadIdx.x;
  const float4 v = *reinterpret_cast<const float4*>(x2 + b * d_in + S * MX_SS + e);
  int cs = a4_put4(v, sc, e, stg, codes_out ? codes_out + b * d_in + S * MX_SS : nullptr);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cs += __shfl_xor(cs, o);
  if ((threadIdx.x & 63) == 0) ipart[threadIdx.x >> 6] = cs;
  __syncthreads();
  a4_store(stg, 1, b, S, nss, xa);
  if (threadIdx.x == 0) {
    asum[b * nss + S] = ipart[0] + ipart[1];
    if (S == 0) {
      ascale[b] = sc;
      if (scale_out) scale_out[b] = sc;
    }
  }
}

// y1[16 tile + v][rows] = scale (s_v (sum_k q_k a_vk - zero sum_k a_vk)) for
// the tile's vectors v and the rows rb * rpw .. + rpw - 1 (rpw a multiple of
// 16) of row block rb; the waves' partial sums meet in LDS (red, nw x rpw x
// 16 floats, sized at launch). Workgroup b runs on XCD b % 8 and takes, in the order that XCD
// receives them, every vector tile of one row block after another: the
// tiles of a row block run together on one XCD and read its codes from HBM
// once, through that XCD's L2. K ranges of RK super-steps; wave w takes
// ranges w, w + waves, ... and holds a range's B operands (all 16 vectors)
// in registers while it streams the rows.
template <int RK>
__global__ __launch_bounds__(1024) void qmatvec_a4_kernel(
    const uint32_t* __restrict__ packed, int rw, const float* __restrict__ scale,
    const float* __restrict__ zero, const uint8_t* __restrict__ xa, const float* __restrict__ ascale,
    const int* __restrict__ asum, int nsum, int64_t nss, int64_t d_out, int nkr, int rpw, int ntiles,
    int64_t batch, float* __restrict__ y1) {
  extern __shared__ float red[];
  __shared__ int vpart[1024];
  __shared__ float vsum[A4_TILE];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const int xcd = blockIdx.x & 7, seq = blockIdx.x >> 3;
  const int tile = seq % ntiles;
  const int64_t rbeg = (int64_t(seq / ntiles) * 8 + xcd) * rpw;
  if (rbeg >= d_out) return;  // the grid is rounded up to whole rounds of 8
  const int nvec = int(min(int64_t(A4_TILE), batch - int64_t(tile) * A4_TILE));
  const int nrows = int(min(int64_t(rpw), d_out - rbeg));
  float* redw = red + w * rpw * A4_TILE;
  for (int i = lane; i < rpw * A4_TILE; i += 64) redw[i] = 0.f;
  const int n = lane & 15, G = lane >> 4;
  const bool bcol = n < nvec;
  const int ntile = (nrows + 15) / 16;
  const int items = ((nkr - 1 - w) / nw + 1) * ntile;
  auto load_a = [&](int it, uint4 (&dst)[RK][2]) {
    const int kr = w + (it / ntile) * nw, t0 = (it % ntile) * 16;
    const int64_t row = rbeg + min(t0 + n, nrows - 1);  // past the end: the last row, not stored
#pragma unroll
    for (int t = 0; t < RK; ++t) {
      const int64_t S = min(int64_t(kr) * RK + t, nss - 1);  // past the end: unused
      const uint4* ap = reinterpret_cast<const uint4*>(packed + row * rw + S * (MX_SS / 16) + G * 4);
      dst[t][0] = ap[0];
      dst[t][1] = ap[4];
    }
  };
  v8i_t bop[RK][4];
  uint4 an[RK][2];
  load_a(0, an);
  // sum_k a_k of each vector from its nsum partial sums: each thread loads
  // one now, to be added up after the rows (integers: any order)
  const int64_t vbase = int64_t(tile) * A4_TILE * nsum;
  const int npart = nvec * nsum;
  const int pre = int(threadIdx.x) < npart ? asum[vbase + threadIdx.x] : 0;
  int cur_kr = -1;
  for (int it = 0; it < items; ++it) {
    const int kr = w + (it / ntile) * nw, t0 = (it % ntile) * 16;
    if (kr != cur_kr) {
      cur_kr = kr;
#pragma unroll
      for (int t = 0; t < RK; ++t) {
        const int64_t S = int64_t(kr) * RK + t;
        const bool ok = bcol && S < nss;
        const uint8_t* bp = xa + ((int64_t(tile) * nss + (S < nss ? S : 0)) * 4) * (64 * 32) + lane * 32;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4* p = reinterpret_cast<const uint4*>(bp + q * (64 * 32));
          const uint4 lo = ok ? p[0] : make_uint4(0u, 0u, 0u, 0u);
          const uint4 hi = ok ? p[1] : make_uint4(0u, 0u, 0u, 0u);
          bop[t][q] = v8i_t{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
        }
      }
    }
    uint4 ac[RK][2];
#pragma unroll
    for (int t = 0; t < RK; ++t) {
      ac[t][0] = an[t][0];
      ac[t][1] = an[t][1];
    }
    if (it + 1 < items) load_a(it + 1, an);
    v4f_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < RK; ++t) {
      if (int64_t(kr) * RK + t >= nss) break;
      const uint32_t wd[8] = {ac[t][0].x, ac[t][0].y, ac[t][0].z, ac[t][0].w,
                              ac[t][1].x, ac[t][1].y, ac[t][1].z, ac[t][1].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t x0 = wd[2 * q], x1 = wd[2 * q + 1];
        const v8i_t aop = {int(x0 & 0x33333333u), int((x0 >> 2) & 0x33333333u),
                           int(x1 & 0x33333333u), int((x1 >> 2) & 0x33333333u), 0, 0, 0, 0};
        // A scale 2^0, B scale 2^1 (E8M0 0x7f, 0x80): undoes the halved codes
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, bop[t][q], acc, 4, 0, 0, 0x7f7f7f7f, 0,
                                                               int(0x80808080u));
      }
    }
    // acc[i] = C[4 G + i][n]: row t0 + 4 G + i, vector n
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = t0 + 4 * G + i;
      if (bcol && r < nrows) redw[r * A4_TILE + n] += acc[i];
    }
  }
  vpart[threadIdx.x] = pre;
  __syncthreads();
  if (int(threadIdx.x) < nvec) {
    int t = 0;
    for (int k = 0; k < nsum; ++k) {
      const int i = int(threadIdx.x) * nsum + k;
      t += i < int(blockDim.x) ? vpart[i] : asum[vbase + i];
    }
    vsum[threadIdx.x] = float(t);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nrows * nvec; i += blockDim.x) {
    const int r = i / nvec, v = i % nvec;
    float acc = 0.f;
    for (int u = 0; u < nw; ++u) acc += red[(u * rpw + r) * A4_TILE + v];
    const int64_t row = rbeg + r, vec = int64_t(tile) * A4_TILE + v;
    y1[vec * d_out + row] = scale[row] * (ascale[vec] * (acc - zero[row] * vsum[v]));
  }
}

// Larger batches: a matrix-core GEMM. A workgroup of 4 waves owns 256 rows x
// 32 vectors (two vector tiles) and streams both operands through a ring of
// three LDS stages, one 512-column super-step each, with
// global_load_lds_dwordx4 (LDS DMA: lane l's 16 bytes land at the
// instruction's base + 16 l). Layouts, one DMA instruction per 1 KB block:
//   codes: block (w, rt, h) holds, for lane l = 16 G + n, the 16 bytes at
//     64 h + 16 G of row 64 w + 16 rt + n's super-step: exactly the A
//     operand half that lane reads, so each wave fills and reads only its own
//     8 blocks and every read is one conflict-free 16-byte read;
//   activations: block (vt, q, h) holds half h of lane l's 32 bytes of vector
//     tile vt, step q.
// Each wave's 4 x 2 grid of 16 x 16 tiles reuses every fragment: 32 MFMAs
// per super-step, one barrier. Workgroups are grouped by XCD as in
// qmatvec_a4_kernel.
constexpr int QG_ROWS = 256, QG_RT = 4, QG_VT = 2;
constexpr int QG_ABYTES = QG_ROWS * (MX_SS / 4);    // 32 KB of codes per super-step
constexpr int QG_STAGE = QG_ABYTES + QG_VT * A4_SSB; // plus 16 KB of activations
constexpr int QG_NST = 3;                           // ring depth
constexpr int QG_DMA = 12;                          // DMA instructions per wave and stage
constexpr int QG_PRE = 8;                           // code-sum partials each thread preloads

__global__ __launch_bounds__(256) void qgemm_a4_kernel(
    const uint32_t* __restrict__ packed, int rw, const float* __restrict__ scale,
    const float* __restrict__ zero, const uint8_t* __restrict__ xa, const float* __restrict__ ascale,
    const int* __restrict__ asum, int nsum, int64_t nss, int64_t d_out, int64_t batch, int nvb,
    float* __restrict__ y1) {
  extern __shared__ __attribute__((aligned(16))) uint8_t ring[];
  __shared__ int vsum[QG_VT * A4_TILE];
  const int t = threadIdx.x, lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const int xcd = blockIdx.x & 7, seq = blockIdx.x >> 3;
  const int vb = seq % nvb;
  const int64_t rbeg = (int64_t(seq / nvb) * 8 + xcd) * QG_ROWS;
  if (rbeg >= d_out) return;  // the grid is rounded up to whole rounds of 8
  const int64_t ntiles = (batch + A4_TILE - 1) / A4_TILE;
  const int64_t v0 = int64_t(vb) * (QG_VT * A4_TILE);
  const int nv = int(min(int64_t(QG_VT * A4_TILE), batch - v0));
  const int n = lane & 15, G = lane >> 4;
  const uint32_t ring_base = uint32_t(reinterpret_cast<uintptr_t>(ring));

  // code sums of this block's vectors: partials loaded now, added at the end
  const int npart = nv * nsum;
  int pre[QG_PRE];
#pragma unroll
  for (int k = 0; k < QG_PRE; ++k) {
    const int i = t + 256 * k;
    pre[k] = i < npart ? asum[v0 * nsum + i] : 0;
  }
  if (t < QG_VT * A4_TILE) vsum[t] = 0;

  // this lane's DMA sources at super-step 0: 8 code blocks (rt, h), then 4
  // activation blocks (vt, q, h) = 4 w .. 4 w + 3 (absent tiles read tile 0:
  // those columns are never stored)
  const uint8_t* src[QG_DMA];
  int64_t step[QG_DMA];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int rt = k >> 1, h = k & 1;
    const int64_t row = min(rbeg + 64 * w + 16 * rt + n, d_out - 1);  // past the end: not stored
    src[k] = reinterpret_cast<const uint8_t*>(packed + row * rw) + 64 * h + 16 * G;
    step[k] = MX_SS / 4;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int blk = 4 * w + k, vt = blk >> 3, q = (blk >> 1) & 3, h = blk & 1;
    const int64_t T = 2 * int64_t(vb) + vt;
    src[8 + k] = xa + (T < ntiles ? T : 0) * nss * A4_SSB + (q * 64 + lane) * 32 + 16 * h;
    step[8 + k] = A4_SSB;
  }
  auto lds_block = [&](int k) {  // LDS byte offset of this wave's DMA block k within a stage
    if (k < 8) return (w * 8 + k) * 1024;
    return QG_ABYTES + (4 * w + (k - 8)) * 1024;
  };
  auto issue = [&](int64_t S) {
    const uint32_t sb = ring_base + uint32_t((S % QG_NST) * QG_STAGE);
#pragma unroll
    for (int k = 0; k < QG_DMA; ++k) a4_dma16(src[k] + S * step[k], sb + uint32_t(lds_block(k)));
  };

  v4f_t acc[QG_RT][QG_VT];
#pragma unroll
  for (int rt = 0; rt < QG_RT; ++rt)
#pragma unroll
    for (int vt = 0; vt < QG_VT; ++vt) acc[rt][vt] = v4f_t{0.f, 0.f, 0.f, 0.f};
  issue(0);
  if (nss > 1) issue(1);
  for (int64_t S = 0; S < nss; ++S) {
    // own DMA of stage S done (stage S + 1 may stay in flight), then every
    // wave's; the barrier also retires all reads of the slot stage S + 2 reuses
    if (S + 1 < nss) a4_wait_vm<QG_DMA>();
    else a4_wait_vm<0>();
    __syncthreads();
    if (S + 2 < nss) issue(S + 2);
    // all of the super-step's fragments first (one LDS latency per step,
    // not one per MFMA group: a SIMD runs a single wave here), then its 32
    // MFMAs back to back
    const uint8_t* st = ring + (S % QG_NST) * QG_STAGE;
    v8i_t b[4][QG_VT];
    uint4 a[QG_RT][2];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int vt = 0; vt < QG_VT; ++vt) {
        const uint8_t* p = st + QG_ABYTES + ((vt * 4 + q) * 2) * 1024 + lane * 16;
        const uint4 lo = *reinterpret_cast<const uint4*>(p);
        const uint4 hi = *reinterpret_cast<const uint4*>(p + 1024);
        b[q][vt] = v8i_t{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
#pragma unroll
    for (int rt = 0; rt < QG_RT; ++rt)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        a[rt][h] = *reinterpret_cast<const uint4*>(st + (w * 8 + 2 * rt + h) * 1024 + lane * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int rt = 0; rt < QG_RT; ++rt) {
        // step q = 2 h + o: words 2 o, 2 o + 1 of half h
        const uint4 x4 = a[rt][q >> 1];
        const uint32_t x0 = (q & 1) ? x4.z : x4.x, x1 = (q & 1) ? x4.w : x4.y;
        const v8i_t aop = {int(x0 & 0x33333333u), int((x0 >> 2) & 0x33333333u),
                           int(x1 & 0x33333333u), int((x1 >> 2) & 0x33333333u), 0, 0, 0, 0};
#pragma unroll
        for (int vt = 0; vt < QG_VT; ++vt)
          acc[rt][vt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aop, b[q][vt], acc[rt][vt], 4, 0, 0,
                                                                         0x7f7f7f7f, 0, int(0x80808080u));
      }
  }
#pragma unroll
  for (int k = 0; k < QG_PRE; ++k)
    if (t + 256 * k < npart) atomicAdd(&vsum[(t + 256 * k) / nsum], pre[k]);
  for (int i = t + 256 * QG_PRE; i < npart; i += 256) atomicAdd(&vsum[i / nsum], asum[v0 * nsum + i]);
  __syncthreads();
  // acc[rt][vt][i] = C[16 rt + 4 G + i][16 vt + n] of the wave's 64 rows
#pragma unroll
  for (int rt = 0; rt < QG_RT; ++rt) {
    const int64_t row0 = rbeg + 64 * w + 16 * rt + 4 * G;
    if (row0 >= d_out) continue;  // d_out % 4 == 0: rows row0 .. row0 + 3 all exist
    const float4 sc = make_float4(scale[row0], scale[row0 + 1], scale[row0 + 2], scale[row0 + 3]);
    const float4 zr = make_float4(zero[row0], zero[row0 + 1], zero[row0 + 2], zero[row0 + 3]);
#pragma unroll
    for (int vt = 0; vt < QG_VT; ++vt) {
      const int v = 16 * vt + n;
      if (v >= nv) continue;
      const float s = ascale[v0 + v], vs = float(vsum[v]);
      const v4f_t a = acc[rt][vt];
      *reinterpret_cast<float4*>(y1 + (v0 + v) * d_out + row0) =
          make_float4(sc.x * (s * (a[0] - zr.x * vs)), sc.y * (s * (a[1] - zr.y * vs)),
                      sc.z * (s * (a[2] - zr.z * vs)), sc.w * (s * (a[3] - zr.w * vs)));
    }
  }
}

struct A4Ws {
  float* x2;
  float* pmax;
  uint8_t* xa;
  float* ascale;
  int* asum;
};

// Sized for any input block (at most d_in / 512 transform chunks per vector);
// x2 is used only when a vector spans several chunks.
A4Ws a4_take(Arena& ar, int64_t d_in, int64_t batch) {
  A4Ws w;
  w.x2 = ar.take<float>(size_t(batch) * d_in);
  w.pmax = ar.take<float>(size_t(batch) * (d_in / MX_SS));
  w.xa = ar.take<uint8_t>(size_t(cdiv(batch, A4_TILE)) * (d_in / MX_SS) * A4_SSB);
  w.ascale = ar.take<float>(size_t(batch));
  w.asum = ar.take<int>(size_t(batch) * (d_in / MX_SS));  // code sums: per vector, or per super-step
  return w;
}

}  // namespace

int64_t packed_row_words(int64_t d_in, int bits) {
  const int64_t w = (d_in * bits + 31) / 32;
  return (w + 3) / 4 * 4;
}

kq_status pack_run(const uint8_t* codes, int64_t d_out, int64_t d_in, int bits, uint32_t* packed,
                   hipStream_t s) {
  const int64_t rw = packed_row_words(d_in, bits);
  const int64_t n = d_out * rw;
  pack_kernel<<<unsigned(cdiv(n, 256)), 256, 0, s>>>(codes, d_out, d_in, bits, rw, packed);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

// The matrix-core path (2-bit codes, one grid per row, d_in % 512 == 0)
bool use_mx(int bits, int group, int64_t d_in) { return bits == 2 && group == 0 && d_in % MX_SS == 0; }

size_t apply_ws_bytes(int64_t d_out, int64_t d_in, int64_t batch) {
  // the larger of the two prepared-input forms, then y1
  Arena a1{nullptr, 0, 0};
  a1.take<uint32_t>(size_t(batch) * (d_in / CODES) * XW);  // prepared input chunks
  Arena a2{nullptr, 0, 0};
  if (d_in % MX_SS == 0) {
    a2.take<uint8_t>(size_t(batch) * (d_in / MX_SS) * MX_BYTES);     // B digits
    a2.take<uint32_t>(size_t(batch) * (d_in / MX_SS) * MX_SCALES);  // B scales
    a2.take<float>(size_t(batch) * (d_in / MX_SS));                 // sums of x2
  }
  Arena ar{nullptr, 0, std::max(a1.used, a2.used)};
  ar.take<float>(size_t(batch) * d_out * mx_planes(d_in));  // y1, or its K-group planes
  return ar.used;
}

kq_status apply_run(const uint32_t* packed, int bits, const float* scale, const float* zero,
                    int group, const float* s_x, const float* s_g, const int8_t* si,
                    const int8_t* so, int64_t bi, int64_t bo, const float* x, int64_t batch,
                    int64_t d_out, int64_t d_in, float* y, Arena& ws, hipStream_t s) {
  const int64_t rw = packed_row_words(d_in, bits);
  const int planes = use_mx(bits, group, d_in) ? int(mx_planes(d_in)) : 1;
  const size_t y1_floats = size_t(batch) * d_out * mx_planes(d_in);
  const size_t front = apply_ws_bytes(d_out, d_in, batch) - y1_floats * sizeof(float);
  char* base = ws.take<char>(front);
  float* y1 = ws.take<float>(y1_floats);
  if (!base || !y1) return fail(KQ_ERR_WORKSPACE, "apply_quantized: workspace too small");
  if (use_mx(bits, group, d_in)) {
    Arena fa{base, front, 0};
    uint8_t* xb = fa.take<uint8_t>(size_t(batch) * (d_in / MX_SS) * MX_BYTES);
    uint32_t* xs = fa.take<uint32_t>(size_t(batch) * (d_in / MX_SS) * MX_SCALES);
    float* xsum = fa.take<float>(size_t(batch) * (d_in / MX_SS));
    if (!xb || !xs || !xsum) return fail(KQ_ERR_WORKSPACE, "apply_quantized: workspace too small");
    KQ_TRY(run_mx(packed, rw, scale, zero, s_x, si, bi, x, batch, d_out, d_in, xb, xs, xsum, y1, s));
  } else {
  uint32_t* xq = reinterpret_cast<uint32_t*>(base);
  const int ngroups = group ? int(d_in / group) : 1;
  const bool grouped = group != 0;
  switch (bits) {
    case 2: KQ_TRY(run_bits<2>(packed, rw, scale, zero, ngroups, grouped, s_x, si, bi, x, batch, d_out, d_in, xq, y1, s)); break;
    case 3: KQ_TRY(run_bits<3>(packed, rw, scale, zero, ngroups, grouped, s_x, si, bi, x, batch, d_out, d_in, xq, y1, s)); break;
    case 4: KQ_TRY(run_bits<4>(packed, rw, scale, zero, ngroups, grouped, s_x, si, bi, x, batch, d_out, d_in, xq, y1, s)); break;
    default: KQ_TRY(run_bits<8>(packed, rw, scale, zero, ngroups, grouped, s_x, si, bi, x, batch, d_out, d_in, xq, y1, s)); break;
  }
  }
  const int64_t Lo = transform_len(d_out, bo);
  const unsigned tout = unsigned(std::max<int64_t>(64, std::min<int64_t>(1024, Lo / 4)));
  with_lgb(ilog2(bo), [&](auto C) {
    transform_out_kernel<decltype(C)::value><<<unsigned(batch * (d_out / Lo)), tout, 0, s>>>(
        y1, d_out, ilog2(Lo), ilog2(bo), so, s_g, float(1.0 / std::sqrt(double(bo))), planes,
        batch * d_out, y);
  });
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}


size_t apply_a4_ws_bytes(int64_t d_out, int64_t d_in, int64_t batch) {
  Arena ar{nullptr, 0, 0};
  a4_take(ar, d_in, batch);
  ar.take<float>(size_t(batch) * d_out);  // y1
  return ar.used;
}

kq_status apply_a4_run(const uint32_t* packed, const float* scale, const float* zero,
                       const float* s_x, const float* s_g, const int8_t* si, const int8_t* so,
                       int64_t bi, int64_t bo, const float* x, int64_t batch, int64_t d_out,
                       int64_t d_in, float clip, float* y, int8_t* codes_out, float* scale_out,
                       Arena& ws, hipStream_t s) {
  const int64_t Li = transform_len(d_in, bi), nparts = d_in / Li, nss = d_in / MX_SS;
  const A4Ws w = a4_take(ws, d_in, batch);
  float* y1 = ws.take<float>(size_t(batch) * d_out);
  if (!w.x2 || !w.pmax || !w.xa || !w.ascale || !w.asum || !y1)
    return fail(KQ_ERR_WORKSPACE, "apply_quantized_a4: workspace too small");
  const unsigned tin = unsigned(std::min<int64_t>(1024, Li / 4));
  const float gain = float(1.0 / std::sqrt(double(bi)));
  if (nparts == 1) {
    with_lgb(ilog2(bi), [&](auto C) {
      transform_in_a4_kernel<true, decltype(C)::value><<<unsigned(batch), tin, 0, s>>>(
          x, d_in, ilog2(Li), ilog2(bi), si, s_x, gain, clip, nullptr, w.pmax, w.xa, w.ascale, w.asum,
          codes_out, scale_out);
    });
    KQ_HIP(hipGetLastError());
  } else {
    with_lgb(ilog2(bi), [&](auto C) {
      transform_in_a4_kernel<false, decltype(C)::value><<<unsigned(batch * nparts), tin, 0, s>>>(
          x, d_in, ilog2(Li), ilog2(bi), si, s_x, gain, clip, w.x2, w.pmax, w.xa, w.ascale, w.asum,
          codes_out, scale_out);
    });
    KQ_HIP(hipGetLastError());
    quantize_a4_kernel<<<unsigned(batch * nss), 128, 0, s>>>(w.x2, w.pmax, int(nparts), d_in, nss, clip,
                                                             w.xa, w.ascale, w.asum, codes_out, scale_out);
    KQ_HIP(hipGetLastError());
  }
  constexpr int RK = 2;
  const int nkr = int(cdiv(nss, RK));
  int nw = std::min(nkr, 16);
  while (nkr % nw) --nw;
  const int64_t rw = packed_row_words(d_in, 2);
  const int64_t ntiles = cdiv(batch, A4_TILE);
  // rows per workgroup: 32 (16 if that leaves < 256 workgroups); with several
  // vector tiles, up to 128 while >= 512 workgroups remain, so that each
  // workgroup's B operands serve more rows
  int rpw = cdiv(d_out, 32) >= 256 ? 32 : 16;
  while (rpw < 128 && cdiv(d_out, 2 * rpw) * ntiles >= 512) rpw *= 2;
  const int64_t nrb = cdiv(d_out, rpw);
  const size_t red_bytes = size_t(nw) * rpw * A4_TILE * sizeof(float);  // <= 128 KB
  KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(qmatvec_a4_kernel<RK>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(red_bytes)));
  const int nsum = nparts == 1 ? 1 : int(nss);
  KQ_TRY(mark_kernel(KQ_OP_APPLY_QUANTIZED_A4, 0, s));
  // the GEMM when its grid gives every CU a workgroup; below that the
  // K-split product keeps more loads in flight
  const int64_t nvb = cdiv(batch, QG_VT * A4_TILE), nrbg = cdiv(d_out, QG_ROWS);
  if (batch > A4_TILE && nvb * nrbg >= 256) {
    constexpr size_t ring_bytes = size_t(QG_NST) * QG_STAGE;  // 144 KB
    KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(qgemm_a4_kernel),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(ring_bytes)));
    qgemm_a4_kernel<<<unsigned(8 * cdiv(nrbg, 8) * nvb), 256, ring_bytes, s>>>(
        packed, int(rw), scale, zero, w.xa, w.ascale, w.asum, nsum, nss, d_out, batch, int(nvb), y1);
  } else {
    qmatvec_a4_kernel<RK><<<unsigned(8 * cdiv(nrb, 8) * ntiles), 64 * nw, red_bytes, s>>>(
        packed, int(rw), scale, zero, w.xa, w.ascale, w.asum, nsum, nss, d_out, nkr, rpw, int(ntiles), batch,
        y1);
  }
  KQ_HIP(hipGetLastError());
  KQ_TRY(mark_kernel(KQ_OP_APPLY_QUANTIZED_A4, 1, s));
  const int64_t Lo = transform_len(d_out, bo);
  const unsigned tout = unsigned(std::max<int64_t>(64, std::min<int64_t>(1024, Lo / 4)));
  with_lgb(ilog2(bo), [&](auto C) {
    transform_out_kernel<decltype(C)::value><<<unsigned(batch * (d_out / Lo)), tout, 0, s>>>(
        y1, d_out, ilog2(Lo), ilog2(bo), so, s_g, float(1.0 / std::sqrt(double(bo))), 1,
        batch * d_out, y);
  });
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

}  // namespace kq
