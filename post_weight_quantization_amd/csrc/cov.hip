// Stage 1: covariances H_X = Xq^T Xq, D = dX^T Xq, H_G = G^T G (scaled by alpha).
//
// KronQ summary (hyper.ai), Method: the Fisher of a linear layer factors under
// K-FAC as H ~ H_X (x) H_G with H_X = E[x x^T] and H_G = E[g g^T]; the GPTAQ
// objective adds the drift term dX X^T. With token-major inputs (one token
// per row), each output is a "TN" product C[i][j] = sum_t A[t][i] B[t][j].
//
// bf16 path (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   * one launch covers every output tile of all three matrices (H_X and H_G
//     lower-triangle tiles only, D full), times `nsplit` token splits;
//     blockIdx % nsplit selects the split so that, with nsplit | 8, all
//     workgroups on one XCD stream the same token range through its L2;
//   * workgroup tile 256 x 256, 4 waves of 128 x 128 (4 x 4 MFMA blocks,
//     256 accumulator registers per lane), 32 tokens per LDS stage;
//   * each thread loads 8 tokens x 4 channels (8 bytes per token row,
//     64 threads cover a 512-byte row segment) and transposes them in
//     registers so LDS holds [channel][token]; an MFMA operand (8 consecutive
//     tokens of one channel) is then one 16-byte LDS read;
//   * for D the A operand is formed on the fly: dX = bf16_rne(X - Xq);
//   * with nsplit == 1 the epilogue applies alpha/beta and mirrors the lower
//     tiles of H_X and H_G into the upper triangle; otherwise partial sums go
//     to scratch and a reduction kernel does the same.
// fp32 path (small workloads): the generic fp32 MFMA GEMM with transposed A.
#include "kq_internal.h"

namespace kq {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int CT = 256;        // output tile edge
constexpr int KS = 32;         // tokens per LDS stage
constexpr int LROW = KS + 8;   // LDS row (uint16): 32 tokens + 16 bytes pad

enum Kind { K_HX = 0, K_D = 1, K_HG = 2 };

struct CovArgs {
  const uint16_t* X;
  const uint16_t* Xq;
  const uint16_t* G;
  int64_t n_tok, d_in, d_out;
  float alpha, beta;
  float* out[3];       // final outputs (direct mode)
  float* part;         // partial sums (split mode): [split][HX | D | HG]
  int64_t part_stride; // floats per split
  int64_t part_off[3]; // offset of each matrix inside one split
  int nt_in, nt_out;   // tiles per dimension
  int tasks[3];        // tiles per matrix (0 when skipped)
  int nsplit;
  int64_t tok_chunk;   // tokens per split (multiple of KS)
};

__device__ inline uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline void tri_decode(int t, int& I, int& J) {
  int i = int((sqrtf(8.f * float(t) + 1.f) - 1.f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  while (i * (i + 1) / 2 > t) --i;
  I = i;
  J = t - i * (i + 1) / 2;
}

struct Rows8 {
  uint2 v[8];  // 8 token rows x 4 channels
};

__device__ inline void load_rows(const uint16_t* __restrict__ src, int64_t ld, int64_t width,
                                 int64_t ch, int64_t t0, int64_t t_end, Rows8& r) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t t = t0 + q;
    uint2 v = make_uint2(0u, 0u);
    if (t < t_end && ch < width) v = *reinterpret_cast<const uint2*>(src + t * ld + ch);
    r.v[q] = v;
  }
}

// transpose 8 tokens x 4 channels into 4 channels x 8 tokens and store to LDS
__device__ inline void store_T(uint16_t* lds_rows, int row0, int tcol, const Rows8& r) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t a = (c < 2) ? r.v[2 * k].x : r.v[2 * k].y;
      const uint32_t b = (c < 2) ? r.v[2 * k + 1].x : r.v[2 * k + 1].y;
      o[k] = (c & 1) ? ((a >> 16) | (b & 0xFFFF0000u)) : ((a & 0xFFFFu) | (b << 16));
    }
    *reinterpret_cast<uint4*>(lds_rows + (row0 + c) * LROW + tcol) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// dX = bf16_rne(X - Xq), elementwise on packed pairs
__device__ inline void drift(Rows8& x, const Rows8& xq) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint32_t w[2] = {x.v[q].x, x.v[q].y};
    const uint32_t wq[2] = {xq.v[q].x, xq.v[q].y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t lo = bf16_rne_bits(bf16_lo(w[h]) - bf16_lo(wq[h]));
      const uint32_t hi = bf16_rne_bits(bf16_hi(w[h]) - bf16_hi(wq[h]));
      w[h] = (lo & 0xFFFFu) | (hi << 16);
    }
    x.v[q] = make_uint2(w[0], w[1]);
  }
}

__global__ __launch_bounds__(256) void cov_bf16_kernel(CovArgs a) {
  __shared__ uint16_t As[2][CT * LROW];
  __shared__ uint16_t Bs[2][CT * LROW];

  const int b = blockIdx.x;
  const int split = b % a.nsplit;
  int tile = b / a.nsplit;
  int kind, I, J;
  if (tile < a.tasks[0]) {
    kind = K_HX;
    tri_decode(tile, I, J);
  } else if ((tile -= a.tasks[0]) < a.tasks[1]) {
    kind = K_D;
    I = tile / a.nt_in;
    J = tile % a.nt_in;
  } else {
    tile -= a.tasks[1];
    kind = K_HG;
    tri_decode(tile, I, J);
  }
  const uint16_t* srcA = kind == K_HG ? a.G : a.Xq;
  const int64_t width = kind == K_HG ? a.d_out : a.d_in;
  const bool same = (kind != K_D) && (I == J);

  const int64_t t_begin = int64_t(split) * a.tok_chunk;
  const int64_t t_end = min(a.n_tok, t_begin + a.tok_chunk);

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int tg = w;            // token group (8 tokens) within a stage
  const int cg = lane;         // channel group (4 channels)
  const int64_t chA = int64_t(I) * CT + 4 * cg;
  const int64_t chB = int64_t(J) * CT + 4 * cg;
  const int wm = (w >> 1) * 128;
  const int wn = (w & 1) * 128;
  const int lr = lane & 31;
  const int lk = lane >> 5;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  Rows8 ra, rb, rx;
  auto load_stage = [&](int64_t tok0) {
    const int64_t t0 = tok0 + 8 * tg;
    load_rows(srcA, width, width, chA, t0, t_end, ra);
    if (kind == K_D) {
      load_rows(a.X, a.d_in, a.d_in, chA, t0, t_end, rx);
      load_rows(a.Xq, a.d_in, a.d_in, chB, t0, t_end, rb);
    } else if (!same) {
      load_rows(srcA, width, width, chB, t0, t_end, rb);
    }
  };
  auto store_stage = [&](int buf) {
    if (kind == K_D) {
      drift(rx, ra);  // rx <- bf16(X - Xq) for the I tile
      store_T(As[buf], 4 * cg, 8 * tg, rx);
    } else {
      store_T(As[buf], 4 * cg, 8 * tg, ra);
    }
    if (!same) store_T(Bs[buf], 4 * cg, 8 * tg, rb);
  };

  if (t_begin < t_end) {
    load_stage(t_begin);
    store_stage(0);
    __syncthreads();
    int buf = 0;
    for (int64_t tok0 = t_begin; tok0 < t_end; tok0 += KS) {
      const bool more = tok0 + KS < t_end;
      if (more) load_stage(tok0 + KS);
      const uint16_t* Ab = As[buf];
      const uint16_t* Bb = same ? As[buf] : Bs[buf];
#pragma unroll
      for (int ks = 0; ks < KS; ks += 16) {
        bf16x8 fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          fa[i] = *reinterpret_cast<const bf16x8*>(Ab + (wm + 32 * i + lr) * LROW + ks + 8 * lk);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          fb[j] = *reinterpret_cast<const bf16x8*>(Bb + (wn + 32 * j + lr) * LROW + ks + 8 * lk);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
      if (more) store_stage(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // acc[i][j][r] holds C[I*CT + wm + 32i + 8(r/4) + 4lk + r%4][J*CT + wn + 32j + lr]
  const int64_t dim = width;
  const int64_t row0 = int64_t(I) * CT + wm;
  const int64_t col0 = int64_t(J) * CT + wn;
  if (a.nsplit == 1) {
    float* C = a.out[kind];
    const float alpha = a.alpha, beta = a.beta;
    const bool mirror = (kind != K_D) && (I != J);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t m = row0 + 32 * i + 8 * q + 4 * lk;  // first of 4 consecutive rows
          const int64_t n = col0 + 32 * j + lr;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = alpha * acc[i][j][4 * q + e];
          if (n < dim) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (m + e < dim) {
                float o = v[e];
                if (beta != 0.f) o += beta * C[(m + e) * dim + n];
                C[(m + e) * dim + n] = o;
              }
            }
            if (mirror && m + 3 < dim) {  // transposed copy: row n, columns m..m+3
              float4* p = reinterpret_cast<float4*>(C + n * dim + m);
              float4 o = make_float4(v[0], v[1], v[2], v[3]);
              if (beta != 0.f) {
                const float4 old = *p;
                o.x += beta * old.x;
                o.y += beta * old.y;
                o.z += beta * old.z;
                o.w += beta * old.w;
              }
              *p = o;
            }
          }
        }
  } else {
    float* P = a.part + split * a.part_stride + a.part_off[kind];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = row0 + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
          const int64_t n = col0 + 32 * j + lr;
          if (m < dim && n < dim) P[m * dim + n] = acc[i][j][r];
        }
  }
}

// Sum the split partials of one matrix, apply alpha/beta, mirror lower tiles
// of symmetric outputs. 64 x 64 tiles; for symmetric matrices only lower
// tiles are scheduled and each writes both (I, J) and (J, I).
__global__ __launch_bounds__(256) void cov_reduce_kernel(const float* __restrict__ part,
                                                         int64_t part_stride, int nsplit,
                                                         float* C, int64_t dim, float alpha,
                                                         float beta, int sym, int ntile) {
  __shared__ float tileT[64][65];
  int I, J;
  if (sym) {
    tri_decode(blockIdx.x, I, J);
  } else {
    I = blockIdx.x / ntile;
    J = blockIdx.x % ntile;
  }
  const int tx = threadIdx.x & 63;
  const int ty = threadIdx.x >> 6;  // 0..3
  const int64_t c = int64_t(J) * 64 + tx;
  for (int rr = ty; rr < 64; rr += 4) {
    const int64_t r = int64_t(I) * 64 + rr;
    float s = 0.f;
    if (r < dim && c < dim) {
      for (int k = 0; k < nsplit; ++k) s += part[k * part_stride + r * dim + c];
      float o = alpha * s;
      if (beta != 0.f) o += beta * C[r * dim + c];
      C[r * dim + c] = o;
      s = alpha * s;
    }
    tileT[rr][tx] = s;
  }
  if (!sym || I == J) return;
  __syncthreads();
  // write the transpose: element (J*64 + rr, I*64 + tx) = tile[tx][rr]
  const int64_t c2 = int64_t(I) * 64 + tx;
  for (int rr = ty; rr < 64; rr += 4) {
    const int64_t r2 = int64_t(J) * 64 + rr;
    if (r2 < dim && c2 < dim) {
      float o = tileT[tx][rr];
      if (beta != 0.f) o += beta * C[r2 * dim + c2];
      C[r2 * dim + c2] = o;
    }
  }
}

// fp32 drift: dX = X - Xq
__global__ void drift_f32_kernel(const float* __restrict__ X, const float* __restrict__ Xq,
                                 float* __restrict__ dX, int64_t n) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += int64_t(gridDim.x) * blockDim.x)
    dX[i] = X[i] - Xq[i];
}

int choose_split(int tiles) {
  // Aim for >= ~4 workgroups per CU (256 CUs); splits stay a divisor of the 8 XCDs.
  int s = 1;
  while (s < 8 && tiles * s < 1024) s *= 2;
  return s;
}

int cov_tiles(int64_t d_in, int64_t d_out, bool hx, bool d, bool hg) {
  const int64_t ti = cdiv(d_in, CT), to = cdiv(d_out, CT);
  int64_t n = 0;
  if (hx) n += ti * (ti + 1) / 2;
  if (d) n += ti * ti;
  if (hg) n += to * (to + 1) / 2;
  return int(n);
}

}  // namespace

size_t cov_ws_bytes(int64_t n_tok, int64_t d_in, int64_t d_out, kq_dtype dt, bool hx, bool d,
                    bool hg) {
  Arena ar{nullptr, 0, 0};
  if (dt == KQ_F32) {
    if (d) ar.take<float>(size_t(n_tok) * d_in);
    return ar.used;
  }
  const int tiles = cov_tiles(d_in, d_out, hx, d, hg);
  const int ns = choose_split(tiles);
  if (ns > 1) {
    const size_t per = (hx ? d_in * d_in : 0) + (d ? d_in * d_in : 0) + (hg ? d_out * d_out : 0);
    ar.take<float>(per * ns);
  }
  return ar.used;
}

kq_status cov_run(const void* X, const void* Xq, const void* G, kq_dtype dt, int64_t n_tok,
                  int64_t d_in, int64_t d_out, float alpha, float beta, float* HX, float* D,
                  float* HG, Arena& ws, hipStream_t s) {
  if (dt == KQ_F32) {
    const float* x = static_cast<const float*>(X);
    const float* xq = static_cast<const float*>(Xq);
    const float* g = static_cast<const float*>(G);
    if (HX) {
      GemmArgs a = gemm_args(xq, d_in, xq, d_in, HX, d_in, d_in, d_in, n_tok, alpha, beta, G_TRANS_A);
      KQ_TRY(gemm_f32(a, s));
    }
    if (D) {
      float* dx = ws.take<float>(size_t(n_tok) * d_in);
      if (!dx) return fail(KQ_ERR_WORKSPACE, "accumulate_cov: workspace too small");
      const int64_t n = n_tok * d_in;
      drift_f32_kernel<<<unsigned(std::min<int64_t>(cdiv(n, 256), 8192)), 256, 0, s>>>(x, xq, dx, n);
      KQ_HIP(hipGetLastError());
      GemmArgs a = gemm_args(dx, d_in, xq, d_in, D, d_in, d_in, d_in, n_tok, alpha, beta, G_TRANS_A);
      KQ_TRY(gemm_f32(a, s));
    }
    if (HG) {
      GemmArgs a = gemm_args(g, d_out, g, d_out, HG, d_out, d_out, d_out, n_tok, alpha, beta, G_TRANS_A);
      KQ_TRY(gemm_f32(a, s));
    }
    return KQ_OK;
  }

  CovArgs a{};
  a.X = static_cast<const uint16_t*>(X);
  a.Xq = static_cast<const uint16_t*>(Xq);
  a.G = static_cast<const uint16_t*>(G);
  a.n_tok = n_tok;
  a.d_in = d_in;
  a.d_out = d_out;
  a.alpha = alpha;
  a.beta = beta;
  a.out[0] = HX;
  a.out[1] = D;
  a.out[2] = HG;
  a.nt_in = int(cdiv(d_in, CT));
  a.nt_out = int(cdiv(d_out, CT));
  a.tasks[0] = HX ? a.nt_in * (a.nt_in + 1) / 2 : 0;
  a.tasks[1] = D ? a.nt_in * a.nt_in : 0;
  a.tasks[2] = HG ? a.nt_out * (a.nt_out + 1) / 2 : 0;
  const int tiles = a.tasks[0] + a.tasks[1] + a.tasks[2];
  if (tiles == 0) return KQ_OK;
  int ns = choose_split(tiles);
  // each split needs at least one stage of tokens
  while (ns > 1 && cdiv(n_tok, ns) < KS) ns /= 2;
  a.nsplit = ns;
  a.tok_chunk = cdiv(cdiv(n_tok, ns), KS) * KS;
  if (ns > 1) {
    int64_t off = 0;
    a.part_off[0] = off;
    if (HX) off += d_in * d_in;
    a.part_off[1] = off;
    if (D) off += d_in * d_in;
    a.part_off[2] = off;
    if (HG) off += d_out * d_out;
    a.part_stride = off;
    a.part = ws.take<float>(size_t(off) * ns);
    if (!a.part) return fail(KQ_ERR_WORKSPACE, "accumulate_cov: workspace too small");
  }
  cov_bf16_kernel<<<unsigned(tiles * ns), 256, 0, s>>>(a);
  KQ_HIP(hipGetLastError());
  if (ns > 1) {
    float* outs[3] = {HX, D, HG};
    const int64_t dims[3] = {d_in, d_in, d_out};
    for (int k = 0; k < 3; ++k) {
      if (!outs[k]) continue;
      const int nt = int(cdiv(dims[k], 64));
      const int sym = k != 1;
      const int blocks = sym ? nt * (nt + 1) / 2 : nt * nt;
      cov_reduce_kernel<<<unsigned(blocks), 256, 0, s>>>(a.part + a.part_off[k], a.part_stride, ns,
                                                         outs[k], dims[k], alpha, beta, sym, nt);
      KQ_HIP(hipGetLastError());
    }
  }
  return KQ_OK;
}

}  // namespace kq
