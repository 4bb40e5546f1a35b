// fp32 MFMA GEMM for gfx950: C = alpha * op(A) op(B) + beta * Cin.
//
// The solver's dense contractions (blocked Cholesky updates, the triangular
// inverse, P = triu_1(D U^T) U, the fold W0 P, the lazy trailing update of the
// column sweep, the objective) all run through this kernel. Triangular
// operands restrict each tile's K range and are masked at load, so the
// algorithmic (triangle-aware) flop counts are what the kernel executes.
//
// Tiling: 128 x 128 output tile per workgroup of 4 waves (2 x 2), each wave a
// 64 x 64 sub-tile held as 2 x 2 v_mfma_f32_32x32x2_f32 accumulators
// (64 AGPRs/lane). K advances 16 per stage through double-buffered LDS stored
// k-major, so the MFMA operand reads (32 consecutive m or n per k) are
// conflict-free. Global loads are float4; all callers pass 16-byte aligned
// pointers and leading dimensions that are multiples of 4.
#include "kq_internal.h"

namespace kq {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int TM = 128;
constexpr int TN = 128;
constexpr int TK = 16;
constexpr int LDSP = TM + 4;  // padded LDS row (floats)

struct Stage {
  float4 a[2];
  float4 b[2];
};

__device__ inline float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

template <bool TA, bool TB>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  const int z = blockIdx.z;
  const float* __restrict__ A = g.A + z * g.strideA;
  const float* __restrict__ B = g.B + z * g.strideB;
  float* C = g.C + z * g.strideC;
  const float* Cin = g.Cin ? g.Cin + z * g.strideC : nullptr;
  const uint32_t fl = g.flags;
  // tile coordinates: dispatch order is blockIdx.x fastest; optionally remap so
  // that the tiles with the longest K range start first
  const int ntn = gridDim.x, ntm = gridDim.y;
  int tn = blockIdx.x, tm = blockIdx.y;
  if (fl & (G_ORDER_NDESC | G_ORDER_MDESC | G_ORDER_DIAG)) {
    const int lin = blockIdx.y * ntn + blockIdx.x;
    if (fl & G_ORDER_NDESC) {
      tn = ntn - 1 - lin / ntm;
      tm = lin % ntm;
    } else if (fl & G_ORDER_MDESC) {
      tm = ntm - 1 - lin / ntn;
      tn = lin % ntn;
    } else {
      // diagonals e = tn - tm from ntn - 1 down to -(ntm - 1)
      int rem = lin;
      int e = ntn - 1;
      for (;; --e) {
        const int len = min(ntn - max(e, 0), ntm - max(-e, 0));
        if (rem < len) break;
        rem -= len;
      }
      tm = max(-e, 0) + rem;
      tn = tm + e;
    }
  }
  const int64_t m0 = int64_t(tm) * TM;
  const int64_t n0 = int64_t(tn) * TN;

  // skip tiles outside the written triangle
  if ((fl & G_OUT_LOWER) && n0 > m0 + TM - 1) return;
  if ((fl & G_OUT_UPPER) && m0 > n0 + TN - 1) return;
  if ((fl & G_OUT_SUPPER) && m0 >= n0 + TN - 1) return;

  const int64_t ko = z * g.kofs;  // global k = local k + ko (for masks)
  int64_t klo = 0, khi = g.K;
  if (fl & G_A_UPPER) klo = max(klo, m0 - ko);
  if (fl & G_A_SUPPER) klo = max(klo, m0 + 1 - ko);
  if (fl & G_A_LOWER) khi = min(khi, m0 + TM - ko);
  if (fl & G_B_UPPER) khi = min(khi, n0 + TN - ko);
  if (fl & G_B_LOWER) klo = max(klo, n0 - ko);
  klo = max<int64_t>(0, klo) & ~int64_t(3);  // keep float4 alignment of k

  __shared__ float As[2][TK][LDSP];
  __shared__ float Bs[2][TK][LDSP];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wm = (w >> 1) * 64;
  const int wn = (w & 1) * 64;
  const int lr = lane & 31;
  const int lk = lane >> 5;

  // load coordinates
  // non-transposed A / transposed B: one row (m or n) per thread pair, 8 k's
  const int r_row = t >> 1;
  const int r_k = (t & 1) * 8;
  // transposed A / non-transposed B: one k per 16 threads, 8 m's (or n's)
  const int c_k = t >> 4;
  const int c_col = (t & 15) * 8;

  auto load = [&](int64_t k0, Stage& st) {
    // A
    if (!TA) {
      const int64_t m = m0 + r_row;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t k = k0 + r_k + 4 * h;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m < g.M && k < khi) v = ld4(A + m * g.lda + k);
        st.a[h] = v;
      }
    } else {
      const int64_t k = k0 + c_k;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t m = m0 + c_col + 4 * h;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m < g.M && k < khi) v = ld4(A + k * g.lda + m);
        st.a[h] = v;
      }
    }
    // B
    if (!TB) {
      const int64_t k = k0 + c_k;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t n = n0 + c_col + 4 * h;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (n < g.N && k < khi) v = ld4(B + k * g.ldb + n);
        st.b[h] = v;
      }
    } else {
      const int64_t n = n0 + r_row;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t k = k0 + r_k + 4 * h;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (n < g.N && k < khi) v = ld4(B + n * g.ldb + k);
        st.b[h] = v;
      }
    }
  };

  auto mask_a = [&](int64_t m, int64_t kg, float v) -> float {
    if ((fl & G_A_UPPER) && kg < m) return 0.f;
    if ((fl & G_A_SUPPER) && kg <= m) return 0.f;
    if ((fl & G_A_LOWER) && kg > m) return 0.f;
    return v;
  };
  auto mask_b = [&](int64_t kg, int64_t n, float v) -> float {
    if ((fl & G_B_UPPER) && kg > n) return 0.f;
    if ((fl & G_B_LOWER) && kg < n) return 0.f;
    return v;
  };
  const bool amask = fl & (G_A_UPPER | G_A_LOWER | G_A_SUPPER);
  const bool bmask = fl & (G_B_UPPER | G_B_LOWER);

  auto store = [&](int64_t k0, const Stage& st, int buf) {
    if (!TA) {
      const int64_t m = m0 + r_row;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float e[4] = {st.a[h].x, st.a[h].y, st.a[h].z, st.a[h].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kk = r_k + 4 * h + q;
          float v = e[q];
          if (amask) v = mask_a(m, k0 + kk + ko, v);
          As[buf][kk][r_row] = v;
        }
      }
    } else {
      const int kk = c_k;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float e[4] = {st.a[h].x, st.a[h].y, st.a[h].z, st.a[h].w};
        if (amask) {
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = mask_a(m0 + c_col + 4 * h + q, k0 + kk + ko, e[q]);
        }
        *reinterpret_cast<float4*>(&As[buf][kk][c_col + 4 * h]) = make_float4(e[0], e[1], e[2], e[3]);
      }
    }
    if (!TB) {
      const int kk = c_k;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float e[4] = {st.b[h].x, st.b[h].y, st.b[h].z, st.b[h].w};
        if (bmask) {
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = mask_b(k0 + kk + ko, n0 + c_col + 4 * h + q, e[q]);
        }
        *reinterpret_cast<float4*>(&Bs[buf][kk][c_col + 4 * h]) = make_float4(e[0], e[1], e[2], e[3]);
      }
    } else {
      const int64_t n = n0 + r_row;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float e[4] = {st.b[h].x, st.b[h].y, st.b[h].z, st.b[h].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kk = r_k + 4 * h + q;
          float v = e[q];
          if (bmask) v = mask_b(k0 + kk + ko, n, v);
          Bs[buf][kk][r_row] = v;
        }
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (klo < khi) {
    Stage st;
    load(klo, st);
    store(klo, st, 0);
    __syncthreads();
    int buf = 0;
    for (int64_t k0 = klo; k0 < khi; k0 += TK) {
      const bool more = k0 + TK < khi;
      if (more) load(k0 + TK, st);
#pragma unroll
      for (int kk = 0; kk < TK; kk += 2) {
        const float a0 = As[buf][kk + lk][wm + lr];
        const float a1 = As[buf][kk + lk][wm + 32 + lr];
        const float b0 = Bs[buf][kk + lk][wn + lr];
        const float b1 = Bs[buf][kk + lk][wn + 32 + lr];
        acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f32_32x32x2f32(a1, b1, acc[1][1], 0, 0, 0);
      }
      if (more) store(k0 + TK, st, buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // epilogue: acc[i][j][r] is element (wm + 32i + 8(r/4) + 4 lk + r%4, wn + 32j + lr)
  const float alpha = g.alpha, beta = g.beta;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
        const int64_t n = n0 + wn + 32 * j + lr;
        if (m >= g.M || n >= g.N) continue;
        if ((fl & G_OUT_LOWER) && n > m) continue;
        if ((fl & G_OUT_UPPER) && n < m) continue;
        if ((fl & G_OUT_SUPPER) && n <= m) continue;
        float v = alpha * acc[i][j][r];
        if (beta != 0.f) v += beta * Cin[m * g.ldc + n];
        C[m * g.ldc + n] = v;
      }
}

__global__ void fill_kernel(float* p, int64_t n, float v) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t step = int64_t(gridDim.x) * blockDim.x;
  for (; i < n; i += step) p[i] = v;
}

__global__ void fill2d_kernel(float* p, int64_t rows, int64_t cols, int64_t ld, float v) {
  const int64_t r = blockIdx.y;
  for (int64_t c = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; c < cols;
       c += int64_t(gridDim.x) * blockDim.x)
    p[r * ld + c] = v;
}

}  // namespace

GemmArgs gemm_args(const float* A, int64_t lda, const float* B, int64_t ldb, float* C, int64_t ldc,
                   int64_t M, int64_t N, int64_t K, float alpha, float beta, uint32_t flags) {
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.Cin = C;
  g.C = C;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.batch = 1;
  g.alpha = alpha;
  g.beta = beta;
  g.flags = flags;
  return g;
}

kq_status gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return KQ_OK;
  if ((g.lda | g.ldb | g.ldc | g.K) & 3)
    return fail(KQ_ERR_SHAPE, "internal gemm: leading dimensions and K must be multiples of 4");
  if ((reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B)) & 15)
    return fail(KQ_ERR_ARG, "internal gemm: operands must be 16-byte aligned");
  dim3 grid(unsigned(cdiv(g.N, TN)), unsigned(cdiv(g.M, TM)), unsigned(g.batch > 0 ? g.batch : 1));
  const bool ta = g.flags & G_TRANS_A, tb = g.flags & G_TRANS_B;
  if (!ta && !tb) gemm_f32_kernel<false, false><<<grid, 256, 0, s>>>(g);
  else if (!ta && tb) gemm_f32_kernel<false, true><<<grid, 256, 0, s>>>(g);
  else if (ta && !tb) gemm_f32_kernel<true, false><<<grid, 256, 0, s>>>(g);
  else gemm_f32_kernel<true, true><<<grid, 256, 0, s>>>(g);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

kq_status fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return KQ_OK;
  const int64_t blocks = std::min<int64_t>(cdiv(n, 256), 8192);
  fill_kernel<<<unsigned(blocks), 256, 0, s>>>(p, n, v);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

kq_status fill_2d(float* p, int64_t rows, int64_t cols, int64_t ld, float v, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return KQ_OK;
  dim3 grid(unsigned(std::min<int64_t>(cdiv(cols, 256), 64)), unsigned(rows));
  fill2d_kernel<<<grid, 256, 0, s>>>(p, rows, cols, ld, v);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

}  // namespace kq
