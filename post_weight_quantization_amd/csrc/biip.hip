// Stage 2: bidirectional incoherence processing (BiIP), and the trace
// reduction of the sensitivity score.
//
// KronQ summary (hyper.ai), Method: W <- S_G W S_X with
// S_X = diag(H_X,jj / ||W_:,j||^2)^(1/4), S_G = diag(H_G,ii / ||W_i,:||^2)^(1/4),
// then W <- U W V^T, H_X <- V H_X V^T, H_G <- U H_G U^T, dX X^T <- V dX X^T V^T
// with random Hadamard U, V. The covariances take the inverse scalings so the
// Kronecker objective is unchanged.
//
// Each two-sided transform M <- A diag(f) M diag(g) B^T (Hadamard blocks,
// signs and scalings folded into f, g) is done as
//   * a row pass: every element is multiplied by f_i g_j and the gain, then
//     each row is transformed blockwise (block b | cols) — rows are
//     contiguous, so a workgroup loads an 8192-element chunk (whole blocks)
//     with float4 loads into LDS, applies radix-8 butterfly passes there and
//     writes it back: one HBM read and one write;
//   * a column pass: the transform along the row index, in passes of at most
//     6 row-index bits. Chunks are nr rows x W columns with nr*W <= 4096 and
//     W >= 64 where the width allows (256-byte row segments). Blocks of up
//     to 64 rows take one pass; larger blocks take an inner pass over the low
//     row-index bits and outer passes over the higher bits (rows at a
//     stride), each a read and a write.
#include "kq_internal.h"
#include "fwht_lds.h"

namespace kq {

namespace {

constexpr int CH = 4096;   // elements per LDS chunk of the column pass
constexpr int CHR = 8192;  // elements per LDS chunk of the row pass (Hadamard blocks up to 8192)
constexpr int CHP = CH + CH / 32;
constexpr int CHRP = CHR + CHR / 32;

// Row pass: chunk = R rows x L cols (R*L = CHR, b | L, L | cols).
// LGB > 0: the Hadamard block's bits fixed at compile time (the workloads'
// 4096 and 8192 blocks); LGB = 0: any block, from lgb.
template <int LGB>
__global__ __launch_bounds__(256) void fwht_rows_kernel(float* M, int64_t rows, int64_t cols,
                                                        int lgL, int lgb, const float* rowf,
                                                        const float* colf, float gain) {
  __shared__ float s[CHRP];
  const int L = 1 << lgL;
  const int R = CHR >> lgL;
  const int64_t chunks_per_row = cols >> lgL;
  const int64_t rc = blockIdx.x / chunks_per_row;
  const int64_t cc = blockIdx.x % chunks_per_row;
  const int64_t r0 = rc * R;
  const int64_t c0 = cc * L;
  const int t = threadIdx.x;
  for (int e = 4 * t; e < CHR; e += 4 * blockDim.x) {
    const int rr = e >> lgL, c = e & (L - 1);
    const int64_t row = r0 + rr;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row < rows) {
      v = *reinterpret_cast<const float4*>(M + row * cols + c0 + c);
      const float f = gain * (rowf ? rowf[row] : 1.f);
      if (colf) {
        const float4 g = *reinterpret_cast<const float4*>(colf + c0 + c);
        v.x *= f * g.x;
        v.y *= f * g.y;
        v.z *= f * g.z;
        v.w *= f * g.w;
      } else {
        v.x *= f;
        v.y *= f;
        v.z *= f;
        v.w *= f;
      }
    }
    s[padi(e)] = v.x;
    s[padi(e + 1)] = v.y;
    s[padi(e + 2)] = v.z;
    s[padi(e + 3)] = v.w;
  }
  __syncthreads();
  lds_fwht_blk<LGB>(s, CHR, lgb);
  for (int e = 4 * t; e < CHR; e += 4 * blockDim.x) {
    const int rr = e >> lgL, c = e & (L - 1);
    const int64_t row = r0 + rr;
    if (row < rows)
      *reinterpret_cast<float4*>(M + row * cols + c0 + c) =
          make_float4(s[padi(e)], s[padi(e + 1)], s[padi(e + 2)], s[padi(e + 3)]);
  }
}

// Row pass for Hadamard blocks of 4096: one block of one row per workgroup
// of 256 threads, 16 elements per thread, the 12 butterfly levels in three
// register stages of 4 with two exchanges through LDS between them (against
// four radix-8 LDS passes plus the staging copies in the kernel above):
//   stage 1: elements 4 t + e + 1024 k (index bits 0, 1 in e and 10, 11 in
//            k), four float4 loads straight from memory, scaling applied;
//   stage 2: elements t % 4 + 4 r + 64 (t / 4) (bits 2..5 in r);
//   stage 3: elements t % 64 + 64 r + 1024 (t / 64) (bits 6..9 in r), stored
//            straight to memory (each store 64 consecutive floats a wave).
// LDS index i sits at i + 4 (i / 64): the float4 writes of stage 1 and the
// reads and writes of stages 2 and 3 are free of bank conflicts.
__device__ inline void bfly16(float (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (!(j & h)) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
}

__device__ __host__ constexpr int pad64(int i) { return i + 4 * (i >> 6); }

__global__ __launch_bounds__(256) void fwht_rows4096_kernel(float* M, int64_t rows, int64_t cols,
                                                            const float* rowf, const float* colf,
                                                            float gain) {
  __shared__ __attribute__((aligned(16))) float sx[pad64(4096)];
  const int64_t nblk = cols >> 12;
  const int64_t row = blockIdx.x / nblk;
  const int64_t c0 = (blockIdx.x % nblk) << 12;
  float* p = M + row * cols + c0;
  const float f = gain * (rowf ? rowf[row] : 1.f);
  const int t = threadIdx.x;
  float v[16];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * t + 1024 * k;
    float4 x = *reinterpret_cast<const float4*>(p + i);
    float4 g = colf ? *reinterpret_cast<const float4*>(colf + c0 + i) : make_float4(1.f, 1.f, 1.f, 1.f);
    v[4 * k] = x.x * f * g.x;
    v[4 * k + 1] = x.y * f * g.y;
    v[4 * k + 2] = x.z * f * g.z;
    v[4 * k + 3] = x.w * f * g.w;
  }
  bfly16(v);
#pragma unroll
  for (int k = 0; k < 4; ++k)
    *reinterpret_cast<float4*>(sx + pad64(4 * t + 1024 * k)) =
        make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
  __syncthreads();
  const int i2 = (t & 3) + 64 * (t >> 2);
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = sx[pad64(i2 + 4 * r)];
  bfly16(v);
#pragma unroll
  for (int r = 0; r < 16; ++r) sx[pad64(i2 + 4 * r)] = v[r];
  __syncthreads();
  const int i3 = (t & 63) + 1024 * (t >> 6);
#pragma unroll
  for (int r = 0; r < 16; ++r) v[r] = sx[pad64(i3 + 64 * r)];
  bfly16(v);
#pragma unroll
  for (int r = 0; r < 16; ++r) p[i3 + 64 * r] = v[r];
}

// Column pass: chunk = nr rows (at row stride rs, starting at a group base)
// x W cols, nr * W <= CH. Transforms over the nr rows.
__global__ __launch_bounds__(256) void fwht_cols_kernel(float* M, int64_t rows, int64_t cols,
                                                        int lgnr, int lgW, int64_t rs,
                                                        int64_t group_rows) {
  __shared__ float s[CHP];
  const int W = 1 << lgW;
  const int n_el = 1 << (lgnr + lgW);
  const int64_t col_chunks = cols >> lgW;
  const int64_t rchunk = blockIdx.x / col_chunks;
  const int64_t c0 = (blockIdx.x % col_chunks) * W;
  // row chunks: groups of group_rows consecutive rows, each holding rs interleaved sets
  const int64_t grp = rchunk / rs;
  const int64_t off = rchunk % rs;
  const int64_t rbase = grp * group_rows + off;
  const int t = threadIdx.x;
  for (int e = 4 * t; e < n_el; e += 4 * blockDim.x) {
    const int a = e >> lgW, c = e & (W - 1);
    const int64_t row = rbase + int64_t(a) * rs;
    const float4 v = *reinterpret_cast<const float4*>(M + row * cols + c0 + c);
    s[padi(e)] = v.x;
    s[padi(e + 1)] = v.y;
    s[padi(e + 2)] = v.z;
    s[padi(e + 3)] = v.w;
  }
  __syncthreads();
  lds_fwht(s, n_el, lgW, lgnr);
  for (int e = 4 * t; e < n_el; e += 4 * blockDim.x) {
    const int a = e >> lgW, c = e & (W - 1);
    const int64_t row = rbase + int64_t(a) * rs;
    *reinterpret_cast<float4*>(M + row * cols + c0 + c) =
        make_float4(s[padi(e)], s[padi(e + 1)], s[padi(e + 2)], s[padi(e + 3)]);
  }
}

// Column pass over 6 row-index bits, 64 rows x 64 columns per workgroup (the
// passes of 4096 blocks), in two register stages with one LDS exchange:
//   stage 1: column t % 64, rows a = t / 64 + 4 j (bits 2..5 of a in j),
//            loaded straight from memory (a wave reads 256 contiguous bytes
//            of a row per load);
//   stage 2: columns 4 (t % 16) .. + 3, rows a = 4 (t / 16) + e (bits 0, 1
//            in e), stored straight to memory as float4.
// Rows are taken as in fwht_cols_kernel: the chunk's row a is
// rbase + a rs.
__global__ __launch_bounds__(256) void fwht_cols64_kernel(float* M, int64_t rows, int64_t cols,
                                                          int64_t rs, int64_t group_rows) {
  constexpr int LD = 68;
  __shared__ __attribute__((aligned(16))) float sx[64 * LD];
  const int64_t col_chunks = cols >> 6;
  const int64_t rchunk = blockIdx.x / col_chunks;
  const int64_t c0 = (blockIdx.x % col_chunks) * 64;
  const int64_t grp = rchunk / rs, off = rchunk % rs;
  const int64_t rbase = grp * group_rows + off;
  const int t = threadIdx.x;
  {
    const int c = t & 63, q = t >> 6;
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = M[(rbase + int64_t(q + 4 * j) * rs) * cols + c0 + c];
    bfly16(v);
#pragma unroll
    for (int j = 0; j < 16; ++j) sx[(q + 4 * j) * LD + c] = v[j];
  }
  __syncthreads();
  const int cg = t & 15, h = t >> 4;
  float4 u[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) u[e] = *reinterpret_cast<const float4*>(&sx[(4 * h + e) * LD + 4 * cg]);
  auto bf = [](float4& a, float4& b) {
    const float4 x = a, y = b;
    a = make_float4(x.x + y.x, x.y + y.y, x.z + y.z, x.w + y.w);
    b = make_float4(x.x - y.x, x.y - y.y, x.z - y.z, x.w - y.w);
  };
  bf(u[0], u[1]);
  bf(u[2], u[3]);
  bf(u[0], u[2]);
  bf(u[1], u[3]);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    *reinterpret_cast<float4*>(M + (rbase + int64_t(4 * h + e) * rs) * cols + c0 + 4 * cg) = u[e];
}

// Sum of squares of each row (one wave per row).
__global__ __launch_bounds__(256) void row_sumsq_kernel(const float* W, int64_t rows, int64_t cols,
                                                        float* out) {
  const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  float acc = 0.f;
  const float* p = W + row * cols;
  for (int64_t c = 4 * lane; c < cols; c += 256) {
    const float4 v = *reinterpret_cast<const float4*>(p + c);
    acc += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) out[row] = acc;
}

// Column sums of squares over a chunk of rows: part[chunk][col].
__global__ __launch_bounds__(256) void col_sumsq_kernel(const float* W, int64_t rows, int64_t cols,
                                                        int64_t rows_per_chunk, float* part) {
  const int64_t c = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t ch = blockIdx.y;
  if (c >= cols) return;
  const int64_t r0 = ch * rows_per_chunk;
  const int64_t r1 = min(rows, r0 + rows_per_chunk);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t r = r0; r < r1; ++r) {
    const float4 v = *reinterpret_cast<const float4*>(W + r * cols + c);
    acc.x += v.x * v.x;
    acc.y += v.y * v.y;
    acc.z += v.z * v.z;
    acc.w += v.w * v.w;
  }
  *reinterpret_cast<float4*>(part + ch * cols + c) = acc;
}

// Scale vectors. For each index k of a side (input or output):
//   sc_k = (H_kk / n2_k)^(1/4)   (1 if H_kk <= 0 or n2_k <= 0)
//   wf_k = sc_k * sign_k       (factor applied to W)
//   hf_k = sign_k / sc_k       (factor applied to both sides of H)
// n2 is the squared norm, summed here from nparts partial rows when given.
__global__ void scales_kernel(const float* H, int64_t n, const float* n2, const float* part,
                              int nparts, const int8_t* sign, float* sc_out, float* wf, float* hf) {
  const int64_t k = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (k >= n) return;
  float nn;
  if (part) {
    nn = 0.f;
    for (int p = 0; p < nparts; ++p) nn += part[p * n + k];
  } else {
    nn = n2[k];
  }
  const float h = H[k * n + k];
  float sc = 1.f;
  if (h > 0.f && nn > 0.f) sc = sqrtf(sqrtf(h / nn));
  const float sg = float(sign[k]);
  if (sc_out) sc_out[k] = sc;
  wf[k] = sc * sg;
  hf[k] = sg / sc;
}

__global__ __launch_bounds__(256) void diag_sum_kernel(const float* H, int64_t n, double* out) {
  __shared__ double red[256];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) acc += double(H[i * n + i]);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

inline int ilog2(int64_t v) {
  int k = 0;
  while ((int64_t(1) << (k + 1)) <= v) ++k;
  return k;
}

}  // namespace

kq_status fwht_rows(float* M, int64_t rows, int64_t cols, int64_t blk, const float* rowf,
                    const float* colf, float gain, hipStream_t s) {
  // L: largest power of two with b | L, L | cols, L <= CH; rows per chunk R = CH / L.
  int64_t L = blk;
  while (L * 2 <= CHR && cols % (L * 2) == 0) L *= 2;
  const int64_t R = CHR / L;
  if (L > CHR) return fail(KQ_ERR_UNSUPPORTED, "biip: Hadamard blocks above %d are not supported", CHR);
  const int64_t chunks = cdiv(rows, R) * (cols / L);
  const int lgb = ilog2(blk);
  if (lgb == 12 && cols % 4096 == 0 && rows * (cols >> 12) <= INT32_MAX) {
    fwht_rows4096_kernel<<<unsigned(rows * (cols >> 12)), 256, 0, s>>>(M, rows, cols, rowf, colf, gain);
  } else if (lgb == 12)
    fwht_rows_kernel<12><<<unsigned(chunks), 256, 0, s>>>(M, rows, cols, ilog2(L), lgb, rowf, colf, gain);
  else if (lgb == 13)
    fwht_rows_kernel<13><<<unsigned(chunks), 256, 0, s>>>(M, rows, cols, ilog2(L), lgb, rowf, colf, gain);
  else
    fwht_rows_kernel<0><<<unsigned(chunks), 256, 0, s>>>(M, rows, cols, ilog2(L), lgb, rowf, colf, gain);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

kq_status fwht_cols(float* M, int64_t rows, int64_t cols, int64_t blk, hipStream_t s) {
  // passes over row-index bits [lo, lo + k) with at most 6 bits each; the
  // chunk width W is the largest power of two <= 4096 / 2^k dividing cols
  if (cols % 4) return fail(KQ_ERR_SHAPE, "biip: column count must be a multiple of 4");
  const int lgb = ilog2(blk);
  int lo = 0;
  while (lo < lgb) {
    const int k = std::min(6, lgb - lo);
    const int64_t rs = int64_t(1) << lo;        // stride between transformed rows
    const int64_t group_rows = rs << k;         // rows covered by one set of strided sets
    int lgW = 12 - k;
    while (lgW > 2 && cols % (int64_t(1) << lgW) != 0) --lgW;
    const int64_t row_chunks = (rows / group_rows) * rs;
    if (k == 6 && cols % 64 == 0) {
      fwht_cols64_kernel<<<unsigned(row_chunks * (cols >> 6)), 256, 0, s>>>(M, rows, cols, rs, group_rows);
    } else {
      const int64_t chunks = row_chunks * (cols >> lgW);
      fwht_cols_kernel<<<unsigned(chunks), 256, 0, s>>>(M, rows, cols, k, lgW, rs, group_rows);
    }
    KQ_HIP(hipGetLastError());
    lo += k;
  }
  return KQ_OK;
}

size_t biip_ws_bytes(int64_t d_out, int64_t d_in) {
  Arena ar{nullptr, 0, 0};
  const int64_t nchunk = std::min<int64_t>(64, d_out);
  ar.take<float>(size_t(nchunk) * d_in);  // column partial sums
  ar.take<float>(d_out);                  // row sums
  ar.take<float>(d_in);                   // s (if caller passes no s_x)
  ar.take<float>(d_out);                  // t
  ar.take<float>(d_in);                   // W column factors
  ar.take<float>(d_out);                  // W row factors
  ar.take<float>(d_in);                   // H_X factors
  ar.take<float>(d_out);                  // H_G factors
  return ar.used;
}

kq_status biip_run(float* W, float* HX, float* D, float* HG, int64_t d_out, int64_t d_in,
                   const int8_t* si, const int8_t* so, int64_t bi, int64_t bo, float* s_x,
                   float* s_g, Arena& ws, hipStream_t s) {
  const int64_t nchunk = std::min<int64_t>(64, d_out);
  float* cpart = ws.take<float>(size_t(nchunk) * d_in);
  float* rsum = ws.take<float>(d_out);
  float* sx = s_x ? s_x : ws.take<float>(d_in);
  float* sg = s_g ? s_g : ws.take<float>(d_out);
  float* wcol = ws.take<float>(d_in);
  float* wrow = ws.take<float>(d_out);
  float* hxf = ws.take<float>(d_in);
  float* hgf = ws.take<float>(d_out);
  if (!cpart || !rsum || !sx || !sg || !wcol || !wrow || !hxf || !hgf)
    return fail(KQ_ERR_WORKSPACE, "biip: workspace too small");

  // squared norms of the unscaled W
  row_sumsq_kernel<<<unsigned(cdiv(d_out, 4)), 256, 0, s>>>(W, d_out, d_in, rsum);
  KQ_HIP(hipGetLastError());
  const int64_t rpc = cdiv(d_out, nchunk);
  col_sumsq_kernel<<<dim3(unsigned(cdiv(d_in, 1024)), unsigned(nchunk)), 256, 0, s>>>(W, d_out, d_in,
                                                                                      rpc, cpart);
  KQ_HIP(hipGetLastError());
  scales_kernel<<<unsigned(cdiv(d_in, 256)), 256, 0, s>>>(HX, d_in, nullptr, cpart, int(nchunk), si,
                                                          sx, wcol, hxf);
  KQ_HIP(hipGetLastError());
  scales_kernel<<<unsigned(cdiv(d_out, 256)), 256, 0, s>>>(HG, d_out, rsum, nullptr, 0, so, sg, wrow,
                                                           hgf);
  KQ_HIP(hipGetLastError());

  const float gw = float(1.0 / std::sqrt(double(bi) * double(bo)));
  KQ_TRY(fwht_rows(W, d_out, d_in, bi, wrow, wcol, gw, s));
  KQ_TRY(fwht_cols(W, d_out, d_in, bo, s));
  KQ_TRY(fwht_rows(HX, d_in, d_in, bi, hxf, hxf, float(1.0 / double(bi)), s));
  KQ_TRY(fwht_cols(HX, d_in, d_in, bi, s));
  if (D) {
    KQ_TRY(fwht_rows(D, d_in, d_in, bi, hxf, hxf, float(1.0 / double(bi)), s));
    KQ_TRY(fwht_cols(D, d_in, d_in, bi, s));
  }
  KQ_TRY(fwht_rows(HG, d_out, d_out, bo, hgf, hgf, float(1.0 / double(bo)), s));
  KQ_TRY(fwht_cols(HG, d_out, d_out, bo, s));
  return KQ_OK;
}

kq_status diag_sum(const float* H, int64_t n, double* out_dev, hipStream_t s) {
  diag_sum_kernel<<<1, 256, 0, s>>>(H, n, out_dev);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

}  // namespace kq
