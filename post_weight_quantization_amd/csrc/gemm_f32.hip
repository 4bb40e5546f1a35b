// fp32 MFMA GEMM for gfx950: C = alpha * op(A) op(B) + beta * Cin.
//
// The solver's dense contractions (blocked Cholesky updates, the triangular
// inverse, P = triu_1(D U^T) U, the fold W0 P, the lazy trailing update of the
// column sweep, the objective) all run through this kernel. Triangular
// operands restrict each tile's K range and are masked at load, so the
// algorithmic (triangle-aware) flop counts are what the kernel executes.
//
// Tiling: T x T output tile per workgroup of 4 waves (2 x 2), T = 64 (each
// wave one 32 x 32 v_mfma_f32_32x32x2_f32 accumulator) or T = 128 (each wave
// 64 x 64 as 2 x 2 accumulators) where an in-place product needs one tile
// across all N columns. K advances 16 per stage through double-buffered LDS stored k-major,
// so the MFMA operand reads (32 consecutive m or n per k) are conflict-free.
// Global loads are float4; all callers pass 16-byte aligned pointers and
// leading dimensions that are multiples of 4.
//
// Tile schedule: the grid is one-dimensional and holds only the tiles that
// write output (a lower or upper triangle of tiles when the output is), so
// no workgroup slot goes to a tile that returns at once. The order flags
// sort the tiles by K range, longest first. Workgroup b runs on XCD b % 8 and
// shares a CU with b + 256, b + 512, ... while they are resident together;
// when the K range varies from tile to tile, every other round of 256 tiles
// is reversed (a "snake"), so a CU that gets one of the longest tiles of a
// round gets one of the shortest of the next.
#include "kq_internal.h"

namespace kq {

typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int TK = 16;

template <int T>
struct Stage {
  float4 a[T / 64];
  float4 b[T / 64];
};

__device__ inline float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }

constexpr uint32_t G_SNAKE = 1u << 31;  // set by the launcher: K range varies by tile
constexpr int ROUND = 256;              // workgroups per round: one per CU

// largest k with k (k + 1) / 2 <= x (x < 2^31: every count here fits 32 bits)
__device__ inline int tri_root(int x) {
  int k = int((sqrtf(8.f * float(x) + 1.f) - 1.f) * 0.5f);
  while (k > 0 && k * (k + 1) / 2 > x) --k;
  while ((k + 1) * (k + 2) / 2 <= x) ++k;
  return k;
}

// (local index) -> (row, column) in a lower triangle of tiles (column <= row)
// of p x q tiles, row by row; with q < p the rows from q on are full
__device__ inline void lower_tile(int loc, int p, int q, int& r, int& c) {
  const int s = min(p, q), t0 = s * (s + 1) / 2;
  if (loc < t0) {
    const int k = tri_root(loc);
    r = k;
    c = loc - k * (k + 1) / 2;
  } else {
    r = s + (loc - t0) / q;
    c = (loc - t0) % q;
  }
}

// tiles of one batch that write output
__host__ __device__ inline int64_t tiles_per_batch(uint32_t fl, int64_t ntm, int64_t ntn) {
  if (fl & G_OUT_LOWER) {
    const int64_t s = ntm < ntn ? ntm : ntn;
    return s * (s + 1) / 2 + (ntm - s) * ntn;
  }
  if (fl & (G_OUT_UPPER | G_OUT_SUPPER)) {
    const int64_t s = ntm < ntn ? ntm : ntn;
    return s * (s + 1) / 2 + (ntn - s) * ntm;
  }
  return ntm * ntn;
}

// blockIdx.x -> (batch, row tile, column tile); the launcher keeps the grid
// below 2^31 tiles
__device__ inline void tile_of(uint32_t fl, int ntm, int ntn, int nb, int& z, int& tm, int& tn) {
  int lin = int(blockIdx.x);
  if (fl & G_SNAKE) {
    const int total = int(gridDim.x);
    const int r = lin / ROUND, o = lin % ROUND;
    const int len = min(ROUND, total - r * ROUND);
    if (r & 1) lin = r * ROUND + (len - 1 - o);
  }
  if (fl & G_OUT_LOWER) {
    const int tpb = int(tiles_per_batch(fl, ntm, ntn));
    z = lin / tpb;
    lower_tile(lin % tpb, ntm, ntn, tm, tn);
    return;
  }
  if (fl & (G_OUT_UPPER | G_OUT_SUPPER)) {
    const int tpb = int(tiles_per_batch(fl, ntm, ntn));
    z = lin / tpb;
    const int loc = lin % tpb;
    if (fl & G_ORDER_DIAG) {
      // diagonals e = tn - tm from ntn - 1 down to 0
      if (ntm == ntn) {
        const int j = tri_root(loc);
        tm = loc - j * (j + 1) / 2;
        tn = tm + (ntn - 1 - j);
      } else {
        int rem = loc;
        int e = ntn - 1;
        for (;; --e) {
          const int len = min(ntn - e, ntm);
          if (rem < len) break;
          rem -= len;
        }
        tm = rem;
        tn = tm + e;
      }
    } else {
      // column by column, ascending
      lower_tile(loc, ntn, ntm, tn, tm);
    }
    return;
  }
  if (fl & (G_ORDER_NDESC | G_ORDER_NASC)) {
    const int per = ntm * nb;
    const int c = lin / per;
    tn = (fl & G_ORDER_NDESC) ? ntn - 1 - c : c;
    z = (lin % per) / ntm;
    tm = lin % ntm;
  } else if (fl & G_ORDER_MDESC) {
    const int per = ntn * nb;
    tm = ntm - 1 - lin / per;
    z = (lin % per) / ntn;
    tn = lin % ntn;
  } else if (fl & G_ORDER_DIAG) {
    // diagonals e = tn - tm from ntn - 1 down to -(ntm - 1)
    const int tpb = ntm * ntn;
    z = lin / tpb;
    int rem = lin % tpb;
    int e = ntn - 1;
    for (;; --e) {
      const int len = min(ntn - max(e, 0), ntm - max(-e, 0));
      if (rem < len) break;
      rem -= len;
    }
    tm = max(-e, 0) + rem;
    tn = tm + e;
  } else {
    const int tpb = ntm * ntn;
    z = lin / tpb;
    tm = (lin % tpb) / ntn;
    tn = lin % ntn;
  }
}

template <bool TA, bool TB, int T>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs g) {
  constexpr int TM = T, TN = T;
  constexpr int LDSP = T + 4;   // padded LDS row (floats)
  constexpr int H = T / 64;     // float4 loads per operand per thread per stage
  constexpr int FD = T / 64;    // 32 x 32 MFMA blocks per wave and dimension
  const uint32_t fl = g.flags;
  int z, tm, tn;
  tile_of(fl, int(cdiv(g.M, TM)), int(cdiv(g.N, TN)), g.batch > 0 ? g.batch : 1, z, tm, tn);
  const float* __restrict__ A = g.A + z * g.strideA;
  const float* __restrict__ B = g.B + z * g.strideB;
  float* C = g.C + z * g.strideC;
  const float* Cin = g.Cin ? g.Cin + z * g.strideC : nullptr;
  const int64_t m0 = int64_t(tm) * TM;
  const int64_t n0 = int64_t(tn) * TN;

  // skip tiles outside the written triangle
  if ((fl & G_OUT_LOWER) && n0 > m0 + TM - 1) return;
  if ((fl & G_OUT_UPPER) && m0 > n0 + TN - 1) return;
  if ((fl & G_OUT_SUPPER) && m0 >= n0 + TN - 1) return;
  if ((fl & G_OUT_NSTART) && n0 < g.ostart + z * g.ostart_ofs) return;
  if ((fl & G_OUT_MSTART) && m0 < g.ostart + z * g.ostart_ofs) return;

  const int64_t ko = g.kbase + z * g.kofs;  // global k = local k + ko (for masks)
  int64_t klo = 0, khi = g.K;
  if (fl & G_A_UPPER) klo = max(klo, m0 - ko);
  if (fl & G_A_SUPPER) klo = max(klo, m0 + 1 - ko);
  if (fl & G_A_LOWER) khi = min(khi, m0 + TM - ko);
  if (fl & G_B_UPPER) khi = min(khi, n0 + TN - ko);
  if (fl & G_B_LOWER) klo = max(klo, n0 - ko);
  klo = max<int64_t>(0, klo) & ~int64_t(3);  // keep float4 alignment of k
  // an empty K range leaves an accumulated output as it is
  if (klo >= khi && g.beta == 1.f && Cin == C) return;

  __shared__ float As[2][TK][LDSP];
  __shared__ float Bs[2][TK][LDSP];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wm = (w >> 1) * (T / 2);
  const int wn = (w & 1) * (T / 2);
  const int lr = lane & 31;
  const int lk = lane >> 5;

  // load coordinates
  // non-transposed A / transposed B: one row (m or n) per 256/T threads,
  // T/16 consecutive k's each
  const int r_row = t / (256 / T);
  const int r_k = (t % (256 / T)) * (T / 16);
  // transposed A / non-transposed B: one k per 16 threads, T/16 m's (or n's)
  const int c_k = t >> 4;
  const int c_col = (t & 15) * (T / 16);

  auto load = [&](int64_t k0, Stage<T>& st) {
    // A
    if (!TA) {
      const int64_t m = m0 + r_row;
#pragma unroll
      for (int h = 0; h < H; ++h) {
        const int64_t k = k0 + r_k + 4 * h;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (m < g.M && k < khi) v = ld4(A + m * g.lda + k);
        st.a[h] = v;
      }
    } else {
      const int64_t k = k0 + c_k;
#pragma unroll
      for (int h = 0; h < H; ++h) {
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
      for (int h = 0; h < H; ++h) {
        const int64_t n = n0 + c_col + 4 * h;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (n < g.N && k < khi) v = ld4(B + k * g.ldb + n);
        st.b[h] = v;
      }
    } else {
      const int64_t n = n0 + r_row;
#pragma unroll
      for (int h = 0; h < H; ++h) {
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

  auto store = [&](int64_t k0, const Stage<T>& st, int buf) {
    if (!TA) {
      const int64_t m = m0 + r_row;
#pragma unroll
      for (int h = 0; h < H; ++h) {
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
      for (int h = 0; h < H; ++h) {
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
      for (int h = 0; h < H; ++h) {
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
      for (int h = 0; h < H; ++h) {
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

  f32x16 acc[FD][FD];
#pragma unroll
  for (int i = 0; i < FD; ++i)
#pragma unroll
    for (int j = 0; j < FD; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (klo < khi) {
    Stage<T> st;
    load(klo, st);
    store(klo, st, 0);
    __syncthreads();
    int buf = 0;
    for (int64_t k0 = klo; k0 < khi; k0 += TK) {
      const bool more = k0 + TK < khi;
      if (more) load(k0 + TK, st);
#pragma unroll
      for (int kk = 0; kk < TK; kk += 2) {
        float a[FD], b[FD];
#pragma unroll
        for (int i = 0; i < FD; ++i) a[i] = As[buf][kk + lk][wm + 32 * i + lr];
#pragma unroll
        for (int j = 0; j < FD; ++j) b[j] = Bs[buf][kk + lk][wn + 32 * j + lr];
#pragma unroll
        for (int i = 0; i < FD; ++i)
#pragma unroll
          for (int j = 0; j < FD; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
      }
      if (more) store(k0 + TK, st, buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // epilogue: acc[i][j][r] is element (wm + 32i + 8(r/4) + 4 lk + r%4, wn + 32j + lr)
  const float alpha = g.alpha, beta = g.beta;
#pragma unroll
  for (int i = 0; i < FD; ++i)
#pragma unroll
    for (int j = 0; j < FD; ++j)
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
  const int64_t nb = g.batch > 0 ? g.batch : 1;
  if ((g.flags & G_C_ALIASES_A) && g.N > 128)
    return fail(KQ_ERR_SHAPE, "internal gemm: an in-place product needs N <= 128");
  // 64-wide tiles: at 5 waves per SIMD they hide latency better than the
  // 128-wide tiles (2 waves per SIMD), also on large dense products, and
  // shorten the longest tile of triangular products; 128-wide tiles only
  // where an in-place product needs one tile across N
  const bool small = !((g.flags & G_C_ALIASES_A) && g.N > 64);
  const int T = small ? 64 : 128;
  GemmArgs ga = g;
  if (g.flags & (G_A_UPPER | G_A_SUPPER | G_A_LOWER | G_B_UPPER | G_B_LOWER)) ga.flags |= G_SNAKE;
  const int64_t tiles = tiles_per_batch(g.flags, cdiv(g.M, T), cdiv(g.N, T)) * nb;
  if (tiles > INT32_MAX) return fail(KQ_ERR_SHAPE, "internal gemm: too many tiles");
  const dim3 grid(static_cast<unsigned>(tiles), 1, 1);
  const bool ta = g.flags & G_TRANS_A, tb = g.flags & G_TRANS_B;
  if (small) {
    if (!ta && !tb) gemm_f32_kernel<false, false, 64><<<grid, 256, 0, s>>>(ga);
    else if (!ta && tb) gemm_f32_kernel<false, true, 64><<<grid, 256, 0, s>>>(ga);
    else if (ta && !tb) gemm_f32_kernel<true, false, 64><<<grid, 256, 0, s>>>(ga);
    else gemm_f32_kernel<true, true, 64><<<grid, 256, 0, s>>>(ga);
  } else {
    if (!ta && !tb) gemm_f32_kernel<false, false, 128><<<grid, 256, 0, s>>>(ga);
    else if (!ta && tb) gemm_f32_kernel<false, true, 128><<<grid, 256, 0, s>>>(ga);
    else if (ta && !tb) gemm_f32_kernel<true, false, 128><<<grid, 256, 0, s>>>(ga);
    else gemm_f32_kernel<true, true, 128><<<grid, 256, 0, s>>>(ga);
  }
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
