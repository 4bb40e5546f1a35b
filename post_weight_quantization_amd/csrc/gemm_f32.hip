// fp32 MFMA GEMM for gfx950: C = alpha * op(A) op(B) + beta * Cin.
//
// The solver's dense contractions (blocked Cholesky updates, the triangular
// inverse, P = triu_1(D U^T) U, the fold W0 P, the lazy trailing update of the
// column sweep, the objective) all run through this kernel. Triangular
// operands restrict each tile's K range and are masked at load, so the
// algorithmic (triangle-aware) flop counts are what the kernel executes.
//
// Kernels: the fp32 matrix-core kernels below (64-, 128- and 256-wide tiles)
// and, for large products with op(A) = A, a kernel that runs the fp32
// product on the bf16 matrix cores as six products of three-term bf16 splits
// (fp32-level accuracy at 6 x 32 instead of 8 x 64 matrix-core cycles per
// 16-deep step of a 32 x 32 block; "three bf16 terms" below).
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

// ------------------------------------------------------------ three bf16 terms
// fp32 products on the bf16 matrix cores. Each fp32 operand element is split
// on the fly into three bf16 terms, x = h + m + l exactly (8 significant bits
// each, by truncation: 24 in all), and a product takes the six term products
// whose weight reaches 2^-16 of the leading one,
//   l_a h_b + m_a m_b + h_a l_b + m_a h_b + h_a m_b + h_a h_b,
// on v_mfma_f32_32x32x16_bf16 with fp32 accumulation (a bf16 x bf16 product
// is exact in fp32). The terms left out are below 2^-24 of the leading one:
// the result carries fp32 rounding, at 6 x 32 matrix-core cycles per 16-deep
// step of a 32 x 32 block against 8 x 64 for v_mfma_f32_32x32x2f32.
//
// 128 x 128 tile per workgroup of 4 waves (2 x 2, each 64 x 64 as 2 x 2
// accumulators), K in stages of 32 through double-buffered LDS. Both operands
// sit in LDS as [row][k] fp32 (row stride 36 floats), so a lane reads the 8
// consecutive k of its row that an MFMA operand takes as two float4 and
// splits them in registers. An operand with K contiguous in memory (A; B when
// stored N x K) is copied as float4; one with N contiguous (B stored K x N)
// is transposed on the way in, each wave reading 16 rows of 64 bytes so that
// its scalar LDS stores fall in 64 different banks. Masks and bounds are
// applied when a stage is stored. A is never transposed here (op(A) = A).
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values -> their three bf16 terms, packed in pairs (element 0 in the
// low half). The terms are truncations: h keeps the top 8 significant bits of
// x, m the top 8 of x - h, and l = x - h - m has at most 8 left, so
// x = h + m + l exactly (each difference is exact in fp32) wherever the
// residuals are normal numbers, i.e. for |x| above about 2^-100.
__device__ inline void split3x2(float x0, float x1, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t b0 = __float_as_uint(x0), b1 = __float_as_uint(x1);
  h = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // {b0 >> 16, b1 >> 16}
  const float r0 = x0 - __uint_as_float(b0 & 0xFFFF0000u);
  const float r1 = x1 - __uint_as_float(b1 & 0xFFFF0000u);
  const uint32_t c0 = __float_as_uint(r0), c1 = __float_as_uint(r1);
  m = __builtin_amdgcn_perm(c1, c0, 0x07060302u);
  const float s0 = r0 - __uint_as_float(c0 & 0xFFFF0000u);
  const float s1 = r1 - __uint_as_float(c1 & 0xFFFF0000u);
  l = __builtin_amdgcn_perm(__float_as_uint(s1), __float_as_uint(s0), 0x07060302u);
}

// 8 consecutive fp32 (two float4) -> three bf16x8 MFMA operands
__device__ inline void split3(const float4& x0, const float4& x1, bf16x8& h, bf16x8& m, bf16x8& l) {
  uint32_t h0, h1, h2, h3, m0, m1, m2, m3, l0, l1, l2, l3;
  split3x2(x0.x, x0.y, h0, m0, l0);
  split3x2(x0.z, x0.w, h1, m1, l1);
  split3x2(x1.x, x1.y, h2, m2, l2);
  split3x2(x1.z, x1.w, h3, m3, l3);
  const u32x4 vh = {h0, h1, h2, h3}, vm = {m0, m1, m2, m3}, vl = {l0, l1, l2, l3};
  h = __builtin_bit_cast(bf16x8, vh);
  m = __builtin_bit_cast(bf16x8, vm);
  l = __builtin_bit_cast(bf16x8, vl);
}

constexpr int XK = 32;       // K per stage
constexpr int XLD = XK + 4;  // LDS row stride (floats)

// XT = 128: 4 waves of 64 x 64 (2 x 2 accumulators); XT = 64: 4 waves of
// 32 x 32 (one accumulator), for triangular products, whose K range differs
// from tile to tile and which need more, shorter tiles to spread evenly.
template <bool TB, int XT>
__global__ __launch_bounds__(256) void gemm_x3_kernel(GemmArgs g) {
  constexpr int FD = XT / 64;   // accumulators per wave and dimension
  constexpr int XH = XT / 32;   // float4 per operand per thread and stage
  __shared__ __attribute__((aligned(16))) float As[2][XT * XLD];
  __shared__ __attribute__((aligned(16))) float Bs[2][XT * XLD];
  const uint32_t fl = g.flags;
  int z, tm, tn;
  tile_of(fl, int(cdiv(g.M, XT)), int(cdiv(g.N, XT)), g.batch > 0 ? g.batch : 1, z, tm, tn);
  const float* __restrict__ A = g.A + z * g.strideA;
  const float* __restrict__ B = g.B + z * g.strideB;
  float* C = g.C + z * g.strideC;
  const float* Cin = g.Cin ? g.Cin + z * g.strideC : nullptr;
  const int64_t m0 = int64_t(tm) * XT;
  const int64_t n0 = int64_t(tn) * XT;
  if ((fl & G_OUT_LOWER) && n0 > m0 + XT - 1) return;
  if ((fl & G_OUT_UPPER) && m0 > n0 + XT - 1) return;
  if ((fl & G_OUT_SUPPER) && m0 >= n0 + XT - 1) return;

  const int64_t ko = g.kbase + z * g.kofs;
  int64_t klo = 0, khi = g.K;
  if (fl & G_A_UPPER) klo = max(klo, m0 - ko);
  if (fl & G_A_SUPPER) klo = max(klo, m0 + 1 - ko);
  if (fl & G_A_LOWER) khi = min(khi, m0 + XT - ko);
  if (fl & G_B_UPPER) khi = min(khi, n0 + XT - ko);
  if (fl & G_B_LOWER) klo = max(klo, n0 - ko);
  klo = max<int64_t>(0, klo) & ~int64_t(3);
  if (klo >= khi && g.beta == 1.f && Cin == C) return;

  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  const int wm = (w >> 1) * (XT / 2), wn = (w & 1) * (XT / 2);
  const int lr = lane & 31, lk = lane >> 5;
  const bool amask = fl & (G_A_UPPER | G_A_LOWER | G_A_SUPPER);
  const bool bmask = fl & (G_B_UPPER | G_B_LOWER);
  const int64_t lda = g.lda, ldb = g.ldb;

  // stage element mapping. K-contiguous operands: float4 h of thread t is row
  // (t + 256 h) / 8, k 4 ((t + 256 h) % 8). B stored K x N: wave w's float4 h
  // covers k 16 (c % 2) + lane / 4 and n 16 (c / 2) + 4 (lane % 4), c = XH w + h.
  float4 ra[XH], rb[XH];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int h = 0; h < XH; ++h) {
      const int idx = t + 256 * h;
      const int row = idx >> 3, k4 = 4 * (idx & 7);
      const int64_t k = k0 + k4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (m0 + row < g.M && k < khi) v = ld4(A + (m0 + row) * lda + k);
      ra[h] = v;
      float4 u = make_float4(0.f, 0.f, 0.f, 0.f);
      if (TB) {
        if (n0 + row < g.N && k < khi) u = ld4(B + (n0 + row) * ldb + k);
      } else {
        const int c = XH * w + h;
        const int kr = 16 * (c & 1) + (lane >> 2), nc = 16 * (c >> 1) + 4 * (lane & 3);
        const int64_t kk = k0 + kr;
        if (n0 + nc < g.N && kk < khi) u = ld4(B + kk * ldb + n0 + nc);
      }
      rb[h] = u;
    }
  };
  auto store = [&](int64_t k0, int buf) {
#pragma unroll
    for (int h = 0; h < XH; ++h) {
      const int idx = t + 256 * h;
      const int row = idx >> 3, k4 = 4 * (idx & 7);
      float4 v = ra[h];
      if (amask) {
        const int64_t m = m0 + row, kg = k0 + k4 + ko;
        float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t kq = kg + q;
          if (((fl & G_A_UPPER) && kq < m) || ((fl & G_A_SUPPER) && kq <= m) ||
              ((fl & G_A_LOWER) && kq > m))
            e[q] = 0.f;
        }
        v = make_float4(e[0], e[1], e[2], e[3]);
      }
      *reinterpret_cast<float4*>(&As[buf][row * XLD + k4]) = v;
      float4 u = rb[h];
      if (TB) {
        if (bmask) {
          const int64_t n = n0 + row, kg = k0 + k4 + ko;
          float e[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t kq = kg + q;
            if (((fl & G_B_UPPER) && kq > n) || ((fl & G_B_LOWER) && kq < n)) e[q] = 0.f;
          }
          u = make_float4(e[0], e[1], e[2], e[3]);
        }
        *reinterpret_cast<float4*>(&Bs[buf][row * XLD + k4]) = u;
      } else {
        const int c = XH * w + h;
        const int kr = 16 * (c & 1) + (lane >> 2), nc = 16 * (c >> 1) + 4 * (lane & 3);
        float e[4] = {u.x, u.y, u.z, u.w};
        if (bmask) {
          const int64_t kg = k0 + kr + ko;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t n = n0 + nc + q;
            if (((fl & G_B_UPPER) && kg > n) || ((fl & G_B_LOWER) && kg < n)) e[q] = 0.f;
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) Bs[buf][(nc + q) * XLD + kr] = e[q];
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

  const int64_t nk = khi > klo ? khi - klo : 0;
  const int nst = int(cdiv(nk, int64_t(XK)));
  if (nst > 0) {
    load(klo);
    store(klo, 0);
    __syncthreads();
  }
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    const bool more = st + 1 < nst;
    if (more) load(klo + int64_t(st + 1) * XK);
#pragma unroll
    for (int ks = 0; ks < XK; ks += 16) {
      bf16x8 ah[FD], am[FD], al[FD], bh[FD], bm[FD], bl[FD];
#pragma unroll
      for (int i = 0; i < FD; ++i) {
        const float* pa = &As[buf][(wm + 32 * i + lr) * XLD + ks + 8 * lk];
        split3(*reinterpret_cast<const float4*>(pa), *reinterpret_cast<const float4*>(pa + 4), ah[i],
               am[i], al[i]);
        const float* pb = &Bs[buf][(wn + 32 * i + lr) * XLD + ks + 8 * lk];
        split3(*reinterpret_cast<const float4*>(pb), *reinterpret_cast<const float4*>(pb + 4), bh[i],
               bm[i], bl[i]);
      }
#pragma unroll
      for (int i = 0; i < FD; ++i)
#pragma unroll
        for (int j = 0; j < FD; ++j) {
          f32x16 c = acc[i][j];
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[i], bh[j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[i], bm[j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bl[j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am[i], bh[j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bm[j], c, 0, 0, 0);
          c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[i], bh[j], c, 0, 0, 0);
          acc[i][j] = c;
        }
    }
    if (more) store(klo + int64_t(st + 1) * XK, buf ^ 1);
    __syncthreads();
  }

  // epilogue: acc[i][j][r] is element (wm + 32 i + 8 (r / 4) + 4 lk + r % 4,
  // wn + 32 j + lr); the reads of C of a block are issued together
  const float alpha = g.alpha, beta = g.beta;
#pragma unroll
  for (int i = 0; i < FD; ++i)
#pragma unroll
    for (int j = 0; j < FD; ++j) {
      float cv[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
        const int64_t n = n0 + wn + 32 * j + lr;
        cv[r] = (beta != 0.f && m < g.M && n < g.N) ? Cin[m * g.ldc + n] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + wm + 32 * i + 8 * (r >> 2) + 4 * lk + (r & 3);
        const int64_t n = n0 + wn + 32 * j + lr;
        if (m >= g.M || n >= g.N) continue;
        if ((fl & G_OUT_LOWER) && n > m) continue;
        if ((fl & G_OUT_UPPER) && n < m) continue;
        if ((fl & G_OUT_SUPPER) && n <= m) continue;
        C[m * g.ldc + n] = alpha * acc[i][j][r] + beta * cv[r];
      }
    }
}

// ------------------------------------------------------------ large tiles
// A 256 x 256 output tile per workgroup of 8 waves (2 x 4); each wave holds
// 128 x 64 as 8 x 4 accumulators of v_mfma_f32_16x16x4f32 (128 AGPRs), so
// two waves share a SIMD. K advances 32 per stage through double-buffered
// LDS, loaded through registers one stage ahead. Per stage a wave issues 256
// MFMAs (8192 cycles of matrix-core work) against 12-48 LDS reads, so the
// stage's loads, stores and barrier are a small fraction of its time.
// An operand whose K index is contiguous in memory (A untransposed, B
// transposed) keeps that layout in LDS ([row][k], row stride 36 floats) and
// is read as one float4 per 16-row block and 16-deep chunk: lane l supplies
// k = 4 (l / 16) + e to the chunk's MFMA e, and the other operand supplies
// the same k. An operand with M or N contiguous keeps [k][row] (row stride
// 260 floats) and is read as one float per MFMA. Masks and bounds are
// applied when a stage is stored to LDS.
// The same design also runs 128 x 128 tiles with 4 waves of 64 x 64 (about
// 74 KB of LDS: two workgroups per CU, whose prologues and epilogues overlap
// each other's K loops).
constexpr int BK = 32;
constexpr int KC_LD = BK + 4;
template <int BT>
struct BigCfg {
  static constexpr int NT = BT == 256 ? 512 : 256;        // threads
  static constexpr int WXN = NT / 128;                     // waves across N (2 rows of waves)
  static constexpr int WM = BT / 2, WN = BT / WXN;         // wave tile (WN = 64)
  static constexpr int NBM = WM / 16, NBN = WN / 16;       // 16 x 16 accumulators per wave
  static constexpr int MC_LD = BT + 4;
  static constexpr int OP_FLOATS = BT * KC_LD > BK * MC_LD ? BT * KC_LD : BK * MC_LD;
  static constexpr size_t LDS = sizeof(float) * size_t(4 * OP_FLOATS);  // 2 operands x 2 buffers
  static constexpr int RSTEP = NT / 8;                     // K-contiguous rows per h step
  static constexpr int Q4 = BT / 4;                        // float4 per M/N-contiguous k-row
};

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <bool TA, bool TB, int BT>
__global__ __launch_bounds__(BigCfg<BT>::NT) void gemm_big_kernel(GemmArgs g) {
  using Cf = BigCfg<BT>;
  constexpr int MC_LD = Cf::MC_LD, OP_FLOATS = Cf::OP_FLOATS, NBM = Cf::NBM, NBN = Cf::NBN;
  constexpr int WM = Cf::WM, WN = Cf::WN, RSTEP = Cf::RSTEP, Q4 = Cf::Q4, NT = Cf::NT;
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const uint32_t fl = g.flags;
  int z, tm, tn;
  tile_of(fl, int(cdiv(g.M, BT)), int(cdiv(g.N, BT)), g.batch > 0 ? g.batch : 1, z, tm, tn);
  const float* __restrict__ A = g.A + z * g.strideA;
  const float* __restrict__ B = g.B + z * g.strideB;
  float* C = g.C + z * g.strideC;
  const float* Cin = g.Cin ? g.Cin + z * g.strideC : nullptr;
  const int64_t m0 = int64_t(tm) * BT;
  const int64_t n0 = int64_t(tn) * BT;

  if ((fl & G_OUT_LOWER) && n0 > m0 + BT - 1) return;
  if ((fl & G_OUT_UPPER) && m0 > n0 + BT - 1) return;
  if ((fl & G_OUT_SUPPER) && m0 >= n0 + BT - 1) return;
  if ((fl & G_OUT_NSTART) && n0 < g.ostart + z * g.ostart_ofs) return;
  if ((fl & G_OUT_MSTART) && m0 < g.ostart + z * g.ostart_ofs) return;

  const int64_t ko = g.kbase + z * g.kofs;
  int64_t klo = 0, khi = g.K;
  if (fl & G_A_UPPER) klo = max(klo, m0 - ko);
  if (fl & G_A_SUPPER) klo = max(klo, m0 + 1 - ko);
  if (fl & G_A_LOWER) khi = min(khi, m0 + BT - ko);
  if (fl & G_B_UPPER) khi = min(khi, n0 + BT - ko);
  if (fl & G_B_LOWER) klo = max(klo, n0 - ko);
  klo = max<int64_t>(0, klo) & ~int64_t(3);
  if (klo >= khi && g.beta == 1.f && Cin == C) return;

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = t >> 6;
  const int wy = w / Cf::WXN, wx = w % Cf::WXN;  // wave rows WM wy, columns WN wx
  const int li = lane & 15, lq = lane >> 4;
  const bool amask = fl & (G_A_UPPER | G_A_LOWER | G_A_SUPPER);
  const bool bmask = fl & (G_B_UPPER | G_B_LOWER);
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

  // staging: four float4 per operand per thread and stage, h = 0..3.
  // K-contiguous operand: row (t / 8) + RSTEP h, k 4 (t % 8); M/N-contiguous:
  // k t / Q4 + 8 h, row 4 (t % Q4). Offsets are 32-bit from the uniform
  // tile origin (a tile's rows times the leading dimension fit in 32 bits).
  const int kq_c = 4 * (t & 7), r_c = t >> 3;        // K-contiguous: k, first row
  const int k_m = t / Q4, r_m = 4 * (t % Q4);        // M/N-contiguous: first k, row
  const int Mrem = int(min<int64_t>(g.M - m0, BT)), Nrem = int(min<int64_t>(g.N - n0, BT));
  const int lda = int(g.lda), ldb = int(g.ldb);
  float4 sa[4], sb[4];
  auto load = [&](int k0) {
    const int krem = int(khi) - k0;
    const float* Ak = TA ? A + int64_t(k0) * g.lda + m0 : A + m0 * g.lda + k0;
    const float* Bk = TB ? B + n0 * g.ldb + k0 : B + int64_t(k0) * g.ldb + n0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float4 va = make_float4(0.f, 0.f, 0.f, 0.f), vb = va;
      if (!TA) {
        if (r_c + RSTEP * h < Mrem && kq_c < krem) va = ld4(Ak + (r_c + RSTEP * h) * lda + kq_c);
      } else {
        if (r_m < Mrem && k_m + 8 * h < krem) va = ld4(Ak + (k_m + 8 * h) * lda + r_m);
      }
      if (TB) {
        if (r_c + RSTEP * h < Nrem && kq_c < krem) vb = ld4(Bk + (r_c + RSTEP * h) * ldb + kq_c);
      } else {
        if (r_m < Nrem && k_m + 8 * h < krem) vb = ld4(Bk + (k_m + 8 * h) * ldb + r_m);
      }
      sa[h] = va;
      sb[h] = vb;
    }
  };
  auto store = [&](int k0, int buf) {
    float* As = lds + (2 * buf) * OP_FLOATS;
    float* Bs = As + OP_FLOATS;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float e[4] = {sa[h].x, sa[h].y, sa[h].z, sa[h].w};
      if (!TA) {
        const int r = r_c + RSTEP * h;
        if (amask) {
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = mask_a(m0 + r, k0 + kq_c + q + ko, e[q]);
        }
        *reinterpret_cast<float4*>(As + r * KC_LD + kq_c) = make_float4(e[0], e[1], e[2], e[3]);
      } else {
        const int kr = k_m + 8 * h;
        if (amask) {
#pragma unroll
          for (int q = 0; q < 4; ++q) e[q] = mask_a(m0 + r_m + q, k0 + kr + ko, e[q]);
        }
        *reinterpret_cast<float4*>(As + kr * MC_LD + r_m) = make_float4(e[0], e[1], e[2], e[3]);
      }
      float f[4] = {sb[h].x, sb[h].y, sb[h].z, sb[h].w};
      if (TB) {
        const int r = r_c + RSTEP * h;
        if (bmask) {
#pragma unroll
          for (int q = 0; q < 4; ++q) f[q] = mask_b(k0 + kq_c + q + ko, n0 + r, f[q]);
        }
        *reinterpret_cast<float4*>(Bs + r * KC_LD + kq_c) = make_float4(f[0], f[1], f[2], f[3]);
      } else {
        const int kr = k_m + 8 * h;
        if (bmask) {
#pragma unroll
          for (int q = 0; q < 4; ++q) f[q] = mask_b(k0 + kr + ko, n0 + r_m + q, f[q]);
        }
        *reinterpret_cast<float4*>(Bs + kr * MC_LD + r_m) = make_float4(f[0], f[1], f[2], f[3]);
      }
    }
  };

  f32x4 acc[NBM][NBN];
#pragma unroll
  for (int i = 0; i < NBM; ++i)
#pragma unroll
    for (int j = 0; j < NBN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const float* As = lds + (2 * buf) * OP_FLOATS;
    const float* Bs = As + OP_FLOATS;
    // one 16-deep chunk at a time keeps the operands of one chunk live
#pragma unroll 1
    for (int kc = 0; kc < BK; kc += 16) {
      float a[NBM][4], b[NBN][4];
#pragma unroll
      for (int i = 0; i < NBM; ++i) {
        const int r = WM * wy + 16 * i + li;
        if (!TA) {
          const float4 v = *reinterpret_cast<const float4*>(As + r * KC_LD + kc + 4 * lq);
          a[i][0] = v.x;
          a[i][1] = v.y;
          a[i][2] = v.z;
          a[i][3] = v.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) a[i][e] = As[(kc + 4 * lq + e) * MC_LD + r];
        }
      }
#pragma unroll
      for (int j = 0; j < NBN; ++j) {
        const int c = WN * wx + 16 * j + li;
        if (TB) {
          const float4 v = *reinterpret_cast<const float4*>(Bs + c * KC_LD + kc + 4 * lq);
          b[j][0] = v.x;
          b[j][1] = v.y;
          b[j][2] = v.z;
          b[j][3] = v.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) b[j][e] = Bs[(kc + 4 * lq + e) * MC_LD + c];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < NBM; ++i)
#pragma unroll
          for (int j = 0; j < NBN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i][e], b[j][e], acc[i][j], 0, 0, 0);
    }
  };

  if (klo < khi) {
    const int k_lo = int(klo), k_hi = int(khi);
    load(k_lo);
    store(k_lo, 0);
    __syncthreads();
    int buf = 0;
    for (int k0 = k_lo; k0 < k_hi; k0 += BK) {
      const bool more = k0 + BK < k_hi;
      if (more) load(k0 + BK);
      compute(buf);
      if (more) store(k0 + BK, buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
  }

  // epilogue through LDS, one half of the tile's rows (one row of waves) at a
  // time: the waves holding that half write their accumulators (acc[i][j][r]
  // is element (WM wy + 16 i + 4 lq + r, WN wx + 16 j + li)), then every
  // thread handles its float4 of it with coalesced, batched reads of C and
  // writes.
  const float alpha = g.alpha, beta = g.beta;
  constexpr int ELD = BT + 4;  // conflict-free column writes, 16-byte rows
  constexpr int PER = WM * BT / 4 / NT;  // float4 per thread per half
  constexpr int BATCH = PER < 8 ? PER : 8;
  auto writes = [&](int64_t m, int64_t n) {
    if (m >= g.M || n >= g.N) return false;
    if ((fl & G_OUT_LOWER) && n > m) return false;
    if ((fl & G_OUT_UPPER) && n < m) return false;
    if ((fl & G_OUT_SUPPER) && n <= m) return false;
    return true;
  };
  const bool vec = ((reinterpret_cast<uintptr_t>(C) | reinterpret_cast<uintptr_t>(Cin ? Cin : C)) & 15) == 0;
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    if (wy == half) {
#pragma unroll
      for (int i = 0; i < NBM; ++i)
#pragma unroll
        for (int j = 0; j < NBN; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) lds[(16 * i + 4 * lq + r) * ELD + WN * wx + 16 * j + li] = acc[i][j][r];
    }
    __syncthreads();
#pragma unroll 1
    for (int q0 = 0; q0 < PER; q0 += BATCH) {
      float4 cv[BATCH];
      if (beta != 0.f) {
#pragma unroll
        for (int q = 0; q < BATCH; ++q) {
          const int idx = t + NT * (q0 + q);
          const int64_t m = m0 + WM * half + idx / Q4, n = n0 + 4 * (idx % Q4);
          cv[q] = make_float4(0.f, 0.f, 0.f, 0.f);
          if (vec && m < g.M && n + 3 < g.N) cv[q] = ld4(Cin + m * g.ldc + n);
        }
      }
#pragma unroll
      for (int q = 0; q < BATCH; ++q) {
        const int idx = t + NT * (q0 + q);
        const int row = idx / Q4, c4 = 4 * (idx % Q4);
        const int64_t m = m0 + WM * half + row, n = n0 + c4;
        const float4 a4 = *reinterpret_cast<const float4*>(lds + row * ELD + c4);
        float v[4] = {alpha * a4.x, alpha * a4.y, alpha * a4.z, alpha * a4.w};
        const bool all = vec && writes(m, n) && writes(m, n + 3) && writes(m, n + 1) && writes(m, n + 2);
        if (all) {
          if (beta != 0.f) {
            v[0] += beta * cv[q].x;
            v[1] += beta * cv[q].y;
            v[2] += beta * cv[q].z;
            v[3] += beta * cv[q].w;
          }
          *reinterpret_cast<float4*>(C + m * g.ldc + n) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (!writes(m, n + e)) continue;
            float o = v[e];
            if (beta != 0.f) o += beta * Cin[m * g.ldc + n + e];
            C[m * g.ldc + n + e] = o;
          }
        }
      }
    }
    __syncthreads();
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

// Tile choice. A round of 256-wide tiles is one per CU (256 CUs); of
// 128-wide tiles two per CU. Measured on the solver's shapes (matrix cores
// busy 0.80-0.85 of the launch for the 256-wide tile, 0.67 for the 128-wide
// one on the same 8192 x 28672 layer), the 256-wide kernel runs a tile's K
// loop at about 0.86 of a CU's fp32 MFMA peak plus about 30 us of prologue
// and epilogue per tile; the 128-wide kernel its two tiles per CU at about
// 0.68 together plus about 10 us; the 64-wide kernel sustains about 0.62 of
// the chip's peak overall. With a uniform K range the
// estimated times are compared; with K ranges that vary by tile the larger
// tiles need at least four rounds to balance.
// set_gemm_tile(64, 128 or 256) forces one kernel where it applies (tests).
thread_local int t_forced_tile = 0;
constexpr int X3_FORCED = 3;  // knob value: the three-term kernel wherever it applies

int choose_tile(const GemmArgs& g, int64_t nb) {
  // in-place products need one tile across N; output starts are given in
  // multiples of the 64-wide tile
  if (g.flags & (G_C_ALIASES_A | G_OUT_NSTART | G_OUT_MSTART)) return 64;
  if (t_forced_tile && t_forced_tile != X3_FORCED) return t_forced_tile;
  if (g.K < 256) return 64;
  const int64_t t256 = tiles_per_batch(g.flags, cdiv(g.M, 256), cdiv(g.N, 256)) * nb;
  const int64_t t128 = tiles_per_batch(g.flags, cdiv(g.M, 128), cdiv(g.N, 128)) * nb;
  const int64_t t64 = tiles_per_batch(g.flags, cdiv(g.M, 64), cdiv(g.N, 64)) * nb;
  if (g.flags & (G_A_UPPER | G_A_SUPPER | G_A_LOWER | G_B_UPPER | G_B_LOWER)) {
    if (t256 >= 4 * 256) return 256;
    if (t128 >= 4 * 512) return 128;
    return 64;
  }
  constexpr double cu_peak = 157.3e12 / 256, chip_peak = 157.3e12;
  const double K = double(g.K);
  const double e256 = double(cdiv(t256, 256)) * (2.0 * 256 * 256 * K / (0.86 * cu_peak) + 30e-6);
  const double e128 = double(cdiv(t128, 512)) * (2.0 * 2 * 128 * 128 * K / (0.68 * cu_peak) + 10e-6);
  const double e64 = 2.0 * double(t64) * 64.0 * 64.0 * K / (0.62 * chip_peak);
  if (e256 <= e128 && e256 <= e64) return 256;
  return e128 <= e64 ? 128 : 64;
}

// The three-term bf16 kernel's tile for a product, or 0 for the fp32
// kernels. It takes products with op(A) = A and a K of at least 256:
//  - with the same K range for every tile, on 128-wide tiles when there are
//    at least 200 of them (below that the 64-wide fp32 tile was faster:
//    136 tiles of 128 took 46 us against 26 us in the kernel trace at 4096);
//  - where a triangular operand makes the K range differ from tile to tile,
//    on 128-wide tiles from 1024 of them (two rounds of two per CU), else on
//    64-wide tiles, whose larger number spreads the long tiles evenly (at
//    4096: P formation 221 + 266 us against 303 + 336 on the 64-wide fp32
//    tile and 303 + 384 on 128-wide ones; the fold, 1024 tiles of 128,
//    490 us against 604 on 64-wide ones).
// The testing knob of set_gemm_tile keeps the fp32 kernels, or forces this
// one (64-wide for triangular products, else 128-wide) wherever it applies.
int x3_tile(const GemmArgs& g, int64_t nb) {
  if (t_forced_tile && t_forced_tile != X3_FORCED) return 0;
  if (g.flags & (G_TRANS_A | G_C_ALIASES_A | G_OUT_NSTART | G_OUT_MSTART)) return 0;
  const bool kmask = g.flags & (G_A_UPPER | G_A_SUPPER | G_A_LOWER | G_B_UPPER | G_B_LOWER);
  if (t_forced_tile == X3_FORCED) return kmask ? 64 : 128;
  if (g.K < 256) return 0;
  const int64_t t128 = tiles_per_batch(g.flags, cdiv(g.M, 128), cdiv(g.N, 128)) * nb;
  if (kmask) return t128 >= 1024 ? 128 : 64;
  return t128 >= 200 ? 128 : 0;
}

template <int BT>
kq_status launch_big(const GemmArgs& ga, int64_t nb, hipStream_t s) {
  // the LDS limit is a per-device function attribute: set it once per device
  static bool attr_set[64] = {};
  int dev = 0;
  KQ_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= 64 || !attr_set[dev]) {
    const int lds = int(BigCfg<BT>::LDS);
    KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_big_kernel<false, false, BT>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_big_kernel<false, true, BT>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_big_kernel<true, false, BT>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(gemm_big_kernel<true, true, BT>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, lds));
    if (dev >= 0 && dev < 64) attr_set[dev] = true;
  }
  const int64_t tiles = tiles_per_batch(ga.flags, cdiv(ga.M, BT), cdiv(ga.N, BT)) * nb;
  if (tiles > INT32_MAX) return fail(KQ_ERR_SHAPE, "internal gemm: too many tiles");
  const dim3 grid(static_cast<unsigned>(tiles), 1, 1);
  constexpr int nt = BigCfg<BT>::NT;
  constexpr size_t lds = BigCfg<BT>::LDS;
  const bool ta = ga.flags & G_TRANS_A, tb = ga.flags & G_TRANS_B;
  if (!ta && !tb) gemm_big_kernel<false, false, BT><<<grid, nt, lds, s>>>(ga);
  else if (!ta && tb) gemm_big_kernel<false, true, BT><<<grid, nt, lds, s>>>(ga);
  else if (ta && !tb) gemm_big_kernel<true, false, BT><<<grid, nt, lds, s>>>(ga);
  else gemm_big_kernel<true, true, BT><<<grid, nt, lds, s>>>(ga);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

void set_gemm_tile(int tile) { t_forced_tile = tile; }

kq_status gemm_f32(const GemmArgs& g, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0) return KQ_OK;
  if ((g.lda | g.ldb | g.ldc | g.K) & 3)
    return fail(KQ_ERR_SHAPE, "internal gemm: leading dimensions and K must be multiples of 4");
  if ((reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B)) & 15)
    return fail(KQ_ERR_ARG, "internal gemm: operands must be 16-byte aligned");
  const int64_t nb = g.batch > 0 ? g.batch : 1;
  if ((g.flags & G_C_ALIASES_A) && g.N > 128)
    return fail(KQ_ERR_SHAPE, "internal gemm: an in-place product needs N <= 128");
  GemmArgs ga = g;
  if (g.flags & (G_A_UPPER | G_A_SUPPER | G_A_LOWER | G_B_UPPER | G_B_LOWER)) ga.flags |= G_SNAKE;
  if (const int xt = x3_tile(g, nb)) {
    const int64_t tiles = tiles_per_batch(g.flags, cdiv(g.M, xt), cdiv(g.N, xt)) * nb;
    if (tiles > INT32_MAX) return fail(KQ_ERR_SHAPE, "internal gemm: too many tiles");
    const dim3 grid(static_cast<unsigned>(tiles), 1, 1);
    const bool tb = g.flags & G_TRANS_B;
    if (xt == 128) {
      if (tb) gemm_x3_kernel<true, 128><<<grid, 256, 0, s>>>(ga);
      else gemm_x3_kernel<false, 128><<<grid, 256, 0, s>>>(ga);
    } else {
      if (tb) gemm_x3_kernel<true, 64><<<grid, 256, 0, s>>>(ga);
      else gemm_x3_kernel<false, 64><<<grid, 256, 0, s>>>(ga);
    }
    KQ_HIP(hipGetLastError());
    return KQ_OK;
  }
  const int tile = choose_tile(g, nb);
  if (tile == 256) return launch_big<256>(ga, nb, s);
  if (tile == 128) return launch_big<128>(ga, nb, s);
  // the 64-wide kernel; its 128-wide form only where an in-place product
  // needs one tile across N
  const bool small = !((g.flags & G_C_ALIASES_A) && g.N > 64);
  const int T = small ? 64 : 128;
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
