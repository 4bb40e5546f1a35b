// Inference with a quantized layer: packed codes and the product with the
// layer in its original basis.
//
// KronQ explainer (gist.science), "Limitazioni": the only inference overhead
// is the orthogonal transforms. The sweep quantizes W' = U S_G W S_X V^T, so
//   y = W^ x = S_G^-1 U^T (W^' (V (S_X^-1 x))),
// with U = blockdiag(H_b / sqrt b) diag(sign_out) and V likewise on the input
// side. One call runs
//   1. x2 = V S_X^-1 x: the row FWHT of the batch with sign_in / s_x folded
//      into its load;
//   2. sums of x2 over every 32-entry chunk (the zero-point term);
//   3. y1 = W^' x2 from the packed codes: a lane takes a chunk of 32 codes of
//      8 rows, with the chunk's x2 values in registers, decodes the codes
//      with constant shifts and accumulates scale (sum q x - zero sum x) per
//      chunk (a grid per row or per 128-column group); the lanes' partial
//      sums meet in a wave reduction;
//   4. y = S_G^-1 diag(sign_out) blockdiag(H_b / sqrt b) y1: the row FWHT of
//      y1, then the output scaling.
// Packing: code j of a row in bits [b j, b j + b) of a little-endian stream
// of 32-bit words, rows padded to a multiple of 4 words.
#include "kq_internal.h"

namespace kq {

namespace {

constexpr int RPW = 8;  // rows per wave in the product
constexpr int BT = 4;   // vectors per pass over the codes

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

// fin = sign_in / s_x; fout = sign_out / s_g
__global__ void factors_kernel(const int8_t* si, const float* s_x, int64_t d_in, const int8_t* so,
                               const float* s_g, int64_t d_out, float* fin, float* fout) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e < d_in) fin[e] = float(si[e]) / s_x[e];
  if (e < d_out) fout[e] = float(so[e]) / s_g[e];
}

// csum[b][c] = sum of x2[b][32c .. 32c + 31]
__global__ void chunk_sum_kernel(const float* __restrict__ x2, int64_t d_in, int64_t nchunk,
                                 int64_t batch, float* __restrict__ csum) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e >= batch * nchunk) return;
  const float4* p = reinterpret_cast<const float4*>(x2 + (e / nchunk) * d_in + (e % nchunk) * 32);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float4 v = p[k];
    s += (v.x + v.y) + (v.z + v.w);
  }
  csum[e] = s;
}

__global__ void post_scale_kernel(const float* __restrict__ y2, const float* __restrict__ fout,
                                  int64_t d_out, int64_t batch, float* __restrict__ y) {
  const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (e < batch * d_out) y[e] = y2[e] * fout[e % d_out];
}

template <int BITS>
__device__ inline uint32_t code_at(const uint32_t (&w)[BITS], int k) {
  const int bit = BITS * k, i = bit >> 5, sh = bit & 31;
  uint32_t v = w[i] >> sh;
  if (sh + BITS > 32) v |= w[i + 1] << (32 - sh);
  return v & ((1u << BITS) - 1);
}

// y1[b0 + b][row] for b < nb (nb <= BT) over all rows; one wave per RPW rows
template <int BITS>
__global__ __launch_bounds__(256) void qmatvec_kernel(const uint32_t* __restrict__ packed,
                                                      int64_t row_words, const float* __restrict__ scale,
                                                      const float* __restrict__ zero, int ngroups,
                                                      int gchunks, const float* __restrict__ x2,
                                                      const float* __restrict__ csum, int64_t d_in,
                                                      int64_t d_out, int b0, int nb,
                                                      float* __restrict__ y1) {
  const int lane = threadIdx.x & 63;
  const int64_t r0 = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * RPW;
  if (r0 >= d_out) return;
  const int64_t nchunk = d_in / 32;
  float acc[RPW][BT];
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) acc[r][b] = 0.f;

  for (int64_t c = lane; c < nchunk; c += 64) {
    float xv[BT][32];
    float cs[BT];
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      const int bb = b < nb ? b0 + b : b0;  // unused slots repeat a valid vector
      const float4* p = reinterpret_cast<const float4*>(x2 + bb * d_in + c * 32);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float4 v = p[k];
        xv[b][4 * k] = v.x;
        xv[b][4 * k + 1] = v.y;
        xv[b][4 * k + 2] = v.z;
        xv[b][4 * k + 3] = v.w;
      }
      cs[b] = csum[bb * nchunk + c];
    }
    const int g = gchunks ? int(c / gchunks) : 0;
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      const int64_t row = min(r0 + r, d_out - 1);
      const uint32_t* src = packed + row * row_words + c * BITS;
      uint32_t w[BITS];
#pragma unroll
      for (int i = 0; i < BITS; ++i) w[i] = src[i];
      float part[BT];
#pragma unroll
      for (int b = 0; b < BT; ++b) part[b] = 0.f;
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        const float q = float(code_at<BITS>(w, k));
#pragma unroll
        for (int b = 0; b < BT; ++b) part[b] = __builtin_fmaf(q, xv[b][k], part[b]);
      }
      const float sc = scale[row * ngroups + g], zr = zero[row * ngroups + g];
#pragma unroll
      for (int b = 0; b < BT; ++b) acc[r][b] += sc * (part[b] - zr * cs[b]);
    }
  }
  // wave sums
#pragma unroll
  for (int r = 0; r < RPW; ++r)
#pragma unroll
    for (int b = 0; b < BT; ++b) {
      float v = acc[r][b];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
      acc[r][b] = v;
    }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < RPW; ++r) {
      if (r0 + r >= d_out) continue;
#pragma unroll
      for (int b = 0; b < BT; ++b)
        if (b < nb) y1[(b0 + b) * d_out + r0 + r] = acc[r][b];
    }
  }
}

template <int BITS>
kq_status launch_qmatvec(const uint32_t* packed, int64_t row_words, const float* scale,
                         const float* zero, int ngroups, int gchunks, const float* x2,
                         const float* csum, int64_t d_in, int64_t d_out, int64_t batch, float* y1,
                         hipStream_t s) {
  const unsigned blocks = unsigned(cdiv(d_out, 4 * RPW));
  for (int64_t b0 = 0; b0 < batch; b0 += BT) {
    const int nb = int(std::min<int64_t>(BT, batch - b0));
    qmatvec_kernel<BITS><<<blocks, 256, 0, s>>>(packed, row_words, scale, zero, ngroups, gchunks, x2,
                                               csum, d_in, d_out, int(b0), nb, y1);
    KQ_HIP(hipGetLastError());
  }
  return KQ_OK;
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

size_t apply_ws_bytes(int64_t d_out, int64_t d_in, int64_t batch) {
  Arena ar{nullptr, 0, 0};
  ar.take<float>(size_t(batch) * d_in);        // x2
  ar.take<float>(size_t(batch) * (d_in / 32));  // chunk sums
  ar.take<float>(size_t(batch) * d_out);       // y1
  ar.take<float>(d_in);                        // sign_in / s_x
  ar.take<float>(d_out);                       // sign_out / s_g
  return ar.used;
}

kq_status apply_run(const uint32_t* packed, int bits, const float* scale, const float* zero,
                    int group, const float* s_x, const float* s_g, const int8_t* si,
                    const int8_t* so, int64_t bi, int64_t bo, const float* x, int64_t batch,
                    int64_t d_out, int64_t d_in, float* y, Arena& ws, hipStream_t s) {
  float* x2 = ws.take<float>(size_t(batch) * d_in);
  float* csum = ws.take<float>(size_t(batch) * (d_in / 32));
  float* y1 = ws.take<float>(size_t(batch) * d_out);
  float* fin = ws.take<float>(d_in);
  float* fout = ws.take<float>(d_out);
  if (!x2 || !csum || !y1 || !fin || !fout) return fail(KQ_ERR_WORKSPACE, "apply_quantized: workspace too small");
  const int64_t mx = std::max(d_in, d_out);
  factors_kernel<<<unsigned(cdiv(mx, 256)), 256, 0, s>>>(si, s_x, d_in, so, s_g, d_out, fin, fout);
  KQ_HIP(hipGetLastError());
  KQ_HIP(hipMemcpyAsync(x2, x, size_t(batch) * d_in * sizeof(float), hipMemcpyDeviceToDevice, s));
  KQ_TRY(fwht_rows(x2, batch, d_in, bi, nullptr, fin, float(1.0 / std::sqrt(double(bi))), s));
  const int64_t nchunk = d_in / 32;
  chunk_sum_kernel<<<unsigned(cdiv(batch * nchunk, 256)), 256, 0, s>>>(x2, d_in, nchunk, batch, csum);
  KQ_HIP(hipGetLastError());
  const int ngroups = group ? int(d_in / group) : 1;
  const int gchunks = group ? group / 32 : 0;
  const int64_t rw = packed_row_words(d_in, bits);
  switch (bits) {
    case 2: KQ_TRY(launch_qmatvec<2>(packed, rw, scale, zero, ngroups, gchunks, x2, csum, d_in, d_out, batch, y1, s)); break;
    case 3: KQ_TRY(launch_qmatvec<3>(packed, rw, scale, zero, ngroups, gchunks, x2, csum, d_in, d_out, batch, y1, s)); break;
    case 4: KQ_TRY(launch_qmatvec<4>(packed, rw, scale, zero, ngroups, gchunks, x2, csum, d_in, d_out, batch, y1, s)); break;
    default: KQ_TRY(launch_qmatvec<8>(packed, rw, scale, zero, ngroups, gchunks, x2, csum, d_in, d_out, batch, y1, s)); break;
  }
  KQ_TRY(fwht_rows(y1, batch, d_out, bo, nullptr, nullptr, float(1.0 / std::sqrt(double(bo))), s));
  post_scale_kernel<<<unsigned(cdiv(batch * d_out, 256)), 256, 0, s>>>(y1, fout, d_out, batch, y);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

}  // namespace kq
