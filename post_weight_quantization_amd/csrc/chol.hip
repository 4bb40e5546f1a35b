// Stage 3: the inverse-Hessian factor of the OBS column update.
//
// KronQ summary (hyper.ai), Method: after quantizing column p the update uses
// the row [H_X^-1]_{p, p+1:}. In the Cholesky form this is row p of the upper
// triangular U with U^T U = (H + delta I)^-1: U_pp U_{p,F} equals row p of the
// inverse of the trailing block H_{p:, p:}.
//
// With J the index reversal, J (H + delta I) J = L L^T (lower Cholesky), so
// H + delta I = R R^T with R = J L J upper and U = R^-1 = J L^-1 J. The
// library therefore:
//   1. writes A = J (H + delta I) J (lower triangle) into U's buffer, with
//      delta = damp * mean(diag H) computed on the device;
//   2. factors A = L L^T in place, right-looking with 128-column blocks: a
//      single-workgroup leaf factors the diagonal block and inverts it, the
//      panel below is solved as a GEMM with that inverse (into a compact
//      temporary, copied back), and the trailing lower triangle takes a
//      rank-128 MFMA update from the compact copy;
//   3. inverts L in place by bottom-up doubling with
//      inv([[A,0],[B,C]]) = [[A^-1, 0], [-C^-1 B A^-1, C^-1]]: every level
//      is two batched, triangle-aware fp32 MFMA GEMMs;
//   4. reverses indices in place to obtain U (upper, zeros below).
// A non-positive (or NaN) pivot is reported through `info`.
#include "kq_internal.h"

#include <climits>
#include <utility>

namespace kq {

namespace {

constexpr int NB = 128;

// A[i][j] = H[n-1-i][n-1-j] + delta [i == j] for i >= j (reads H's upper triangle)
__global__ void reverse_damp_kernel(const float* __restrict__ H, int64_t n, const double* dsum,
                                    float damp, float* __restrict__ A) {
  const int64_t i = blockIdx.y;
  const float delta = float(double(damp) * (*dsum) / double(n));
  for (int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; j <= i;
       j += int64_t(gridDim.x) * blockDim.x) {
    float v = H[(n - 1 - i) * n + (n - 1 - j)];
    if (i == j) v += delta;
    A[i * n + j] = v;
  }
}

// ---------------------------------------------------------------- the leaf
// Factor the NB x NB diagonal block at (k0, k0) of A (ld n) in place (lower,
// zeros written above the diagonal) and write its inverse to Dinv (NB x NB,
// zeros above the diagonal). One workgroup of 4 waves; the block lives in LDS.
// Per 32-column panel:
//  * wave 0 factors the 32 x 32 diagonal block and inverts it in registers
//    (leaf_diag32), with no barrier or LDS access inside the 32 column steps;
//  * the waves solve the rows below as a product with the inverse
//    (L21 = A21 L11^-T) and take the rank-32 update of the trailing lower
//    triangle, in 32 x 32 blocks on the matrix cores;
// then the off-diagonal blocks of the inverse X_ip = -X_ii sum_k L_ik X_kp,
// one block column per wave, also on the matrix cores.
constexpr int LS = NB + 4;  // LDS row stride (floats), keeps float4 alignment

__device__ inline float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ inline void wave_lds_fence() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Broadcast of lane J of each 16-lane row (DPP row_newbcast) to that row.
template <int J>
__device__ inline float bc16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + J,
                                                            0xF, 0xF, true));
}

// x[J + 1 + K] += nmm * (entry (J + 1 + K, J): lane J + 1 + K's x[J], the
// symmetric mirror of row J's entry), nmm = minus the row's multiplier
template <int J, int... K>
__device__ inline void chol16_upd_x(float (&x)[16], float nmm, std::integer_sequence<int, K...>) {
  ((x[J + 1 + K] = __builtin_fmaf(bc16<J + 1 + K>(x[J]), nmm, x[J + 1 + K])), ...);
}

// y[K] += nmm * (row J of Y: lane J's y[K]), K <= J
template <int J, int... K>
__device__ inline void chol16_upd_y(float (&y)[16], float nmm, std::integer_sequence<int, K...>) {
  ((y[K] = __builtin_fmaf(bc16<J>(y[K]), nmm, y[K])), ...);
}

// Step J of the 16 x 16 elimination: the pivot is lane J's x[J]; the rows
// below take multipliers x_r[J] / piv, and the same row operations apply to
// Y. Only the lower triangle of the block is ever read.
template <int J>
struct Chol16 {
  __device__ static void run(float (&x)[16], float (&y)[16], float (&dv)[16], int r, int col0,
                             int* info) {
    float piv = bc16<J>(x[J]);
    if (!(piv > 0.f)) {  // non-positive or NaN pivot
      if ((threadIdx.x & 63) == 0) atomicMin(info, col0 + J + 1);
      piv = 1.f;
    }
    const float nmm = r > J ? -(x[J] * __builtin_amdgcn_rcpf(piv)) : 0.f;  // minus the multiplier
    chol16_upd_x<J>(x, nmm, std::make_integer_sequence<int, 15 - J>{});
    chol16_upd_y<J>(y, nmm, std::make_integer_sequence<int, J + 1>{});
    dv[J] = __builtin_amdgcn_sqrtf(piv);  // 1-ulp hardware square root
    Chol16<J + 1>::run(x, y, dv, r, col0, info);
  }
};
template <>
struct Chol16<16> {
  __device__ static void run(float (&)[16], float (&)[16], float (&)[16], int, int, int*) {}
};

// Cholesky and inverse of the 16 x 16 block at (R0, R0) of As (row stride
// LS), one row per lane (lane r % 16 holds row r; the four 16-lane rows of
// the wave hold copies): A = L_u D L_u^T by elimination with Y = L_u^-1,
// then L[r][k] = x_r[k] / sqrt(piv_k) and L^-1 = D^(-1/2) Y. Lanes below 16
// write L (zeros above the diagonal) to As and L^-1 to Xs.
__device__ inline void chol16_block(float* As, float* Xs, int R0, int col0, int* info) {
  const int r = threadIdx.x & 15;
  float x[16], y[16], dv[16];
  const float* row = As + (R0 + r) * LS + R0;
#pragma unroll
  for (int k = 0; k < 16; k += 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + k);
    x[k] = v.x;
    x[k + 1] = v.y;
    x[k + 2] = v.z;
    x[k + 3] = v.w;
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) y[k] = k == r ? 1.f : 0.f;
  Chol16<0>::run(x, y, dv, r, col0, info);
  float dr = dv[0];
#pragma unroll
  for (int k = 1; k < 16; ++k) dr = r == k ? dv[k] : dr;
  const float idr = __builtin_amdgcn_rcpf(dr);
  if ((threadIdx.x & 63) < 16) {
    float* lrow = As + (R0 + r) * LS + R0;
    float* xrow = Xs + (R0 + r) * LS + R0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      lrow[k] = k < r ? x[k] * __builtin_amdgcn_rcpf(dv[k]) : (k == r ? dr : 0.f);
      xrow[k] = k <= r ? y[k] * idr : 0.f;
    }
  }
}

// Cholesky of the 32 x 32 block at (C0, C0) of As and its inverse (wave 0):
// two 16 x 16 factors with 16 x 16 products between them,
//   L11 X11 = chol(A11), L21 = A21 X11^T, A22 -= L21 L21^T,
//   L22 X22 = chol(A22), X21 = -X22 (L21 X11).
// The products take lane l = (r, column group): row r = l % 16, columns
// 4 (l / 16) .. + 3, reading their operands from LDS.
__device__ void leaf_diag32(float* As, float* Xs, int64_t k0, int* info, int C0) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15, c0 = 4 * (lane >> 4);
  const int col0 = int(k0) + C0;
  chol16_block(As, Xs, C0, col0, info);
  wave_lds_fence();
  // L21[r][c] = sum_{k <= c} A21[r][k] X11[c][k]
  float a[16];
  {
    const float* arow = As + (C0 + 16 + r) * LS + C0;
#pragma unroll
    for (int k = 0; k < 16; ++k) a[k] = arow[k];
  }
  float l21[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float* xr = Xs + (C0 + c0 + q) * LS + C0;
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t = __builtin_fmaf(a[k], xr[k], t);  // X11 is zero above its diagonal
    l21[q] = t;
  }
  wave_lds_fence();
#pragma unroll
  for (int q = 0; q < 4; ++q) As[(C0 + 16 + r) * LS + C0 + c0 + q] = l21[q];
  wave_lds_fence();
  // A22[r][c] -= sum_k L21[r][k] L21[c][k] (lower triangle used)
  {
    float lr[16];
    const float* lrow = As + (C0 + 16 + r) * LS + C0;
#pragma unroll
    for (int k = 0; k < 16; ++k) lr[k] = lrow[k];
    float upd[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float* lc = As + (C0 + 16 + c0 + q) * LS + C0;
      float t = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) t = __builtin_fmaf(lr[k], lc[k], t);
      upd[q] = t;
    }
    wave_lds_fence();
#pragma unroll
    for (int q = 0; q < 4; ++q) As[(C0 + 16 + r) * LS + C0 + 16 + c0 + q] -= upd[q];
  }
  wave_lds_fence();
  chol16_block(As, Xs, C0 + 16, col0 + 16, info);
  wave_lds_fence();
  // T = L21 X11 (T[r][c] = sum_{k >= c} L21[r][k] X11[k][c]), then X21 = -X22 T
  {
    float lr[16];
    const float* lrow = As + (C0 + 16 + r) * LS + C0;
#pragma unroll
    for (int k = 0; k < 16; ++k) lr[k] = lrow[k];
    float t4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float t = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) t = __builtin_fmaf(lr[k], Xs[(C0 + k) * LS + C0 + c0 + q], t);
      t4[q] = t;
    }
    // T goes to the unused upper-right block of Xs (rows 0..15, columns 16..31)
#pragma unroll
    for (int q = 0; q < 4; ++q) Xs[(C0 + r) * LS + C0 + 16 + c0 + q] = t4[q];
    wave_lds_fence();
    float xr[16];
    const float* x22 = Xs + (C0 + 16 + r) * LS + C0 + 16;
#pragma unroll
    for (int k = 0; k < 16; ++k) xr[k] = x22[k];  // zero above the diagonal
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float t = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) t = __builtin_fmaf(xr[k], Xs[(C0 + k) * LS + C0 + 16 + c0 + q], t);
      o[q] = -t;
    }
    wave_lds_fence();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      Xs[(C0 + 16 + r) * LS + C0 + c0 + q] = o[q];
      Xs[(C0 + r) * LS + C0 + 16 + c0 + q] = 0.f;  // upper-right of X back to zero
      As[(C0 + r) * LS + C0 + 16 + c0 + q] = 0.f;  // and of L
    }
  }
}

// ---- 32 x 32 block products on the matrix cores (one wave each).
// v_mfma_f32_32x32x2_f32: lane l supplies A[l % 32][k + l / 32] and
// B[k + l / 32][l % 32]; accumulator element r of lane l is
// C[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
typedef float f32x16 __attribute__((ext_vector_type(16)));

// acc += sgn * A op(B): A is 32 x K (rows at ld LS); TB: B holds B[c][k]
// (op = transpose), else B[k][c].
template <bool TB>
__device__ inline void mma32(const float* A, const float* B, int K, float sgn, f32x16& acc) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll 4
  for (int k = 0; k < K; k += 2) {
    const float a = sgn * A[lr * LS + k + lk];
    const float bv = TB ? B[lr * LS + k + lk] : B[(k + lk) * LS + lr];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv, acc, 0, 0, 0);
  }
}

__device__ inline void acc_load(const float* C, f32x16& acc) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = C[(8 * (r >> 2) + 4 * lk + (r & 3)) * LS + lr];
}

__device__ inline void acc_store(float* C, const f32x16& acc) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lk = lane >> 5;
#pragma unroll
  for (int r = 0; r < 16; ++r) C[(8 * (r >> 2) + 4 * lk + (r & 3)) * LS + lr] = acc[r];
}

__device__ inline void acc_zero(f32x16& acc) {
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
}

// Rows C0 + 32 .. NB - 1 of panel columns C0 .. C0 + 31:
// L21 = A21 L11^-T, i.e. L21[r][c] = sum_k A21[r][k] X11[c][k]. Wave w takes
// block row w (in place: a wave reads only the rows it writes).
__device__ void leaf_trsm_below(float* As, const float* Xs, int C0) {
  const int w = threadIdx.x >> 6;
  const int r0 = C0 + 32;
  if (w >= (NB - r0) / 32) return;
  f32x16 acc;
  acc_zero(acc);
  float* blk = As + (r0 + 32 * w) * LS + C0;
  mma32<true>(blk, Xs + C0 * LS + C0, 32, 1.f, acc);
  acc_store(blk, acc);
}

// Trailing lower triangle, rows and columns >= r0: As[r][c] -= sum_k
// As[r][c0 + k] As[c][c0 + k] (k < 32), in 32 x 32 blocks over the waves.
__device__ void leaf_syrk(float* As, int c0, int r0) {
  const int w = threadIdx.x >> 6;
  const int nb = (NB - r0) / 32;
  for (int t = w, i = 0, j = 0, idx = 0; idx < nb * (nb + 1) / 2; ++idx) {
    // block idx -> (i, j), j <= i, row by row
    if (idx > 0) {
      if (j < i) ++j;
      else { ++i; j = 0; }
    }
    if (idx % 4 != t) continue;
    f32x16 acc;
    float* C = As + (r0 + 32 * i) * LS + r0 + 32 * j;
    acc_load(C, acc);
    mma32<true>(As + (r0 + 32 * i) * LS + c0, As + (r0 + 32 * j) * LS + c0, 32, -1.f, acc);
    acc_store(C, acc);
  }
}

__global__ __launch_bounds__(256) void leaf_kernel(float* A, int64_t n, int64_t k0, float* Dinv,
                                                   int* info) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* As = sm;                    // NB x LS: the block, then L
  float* Xs = sm + NB * LS;          // NB x LS: the inverse
  const int t = threadIdx.x;
  const int w = t >> 6;
  float* base = A + k0 * n + k0;
  {
    // the diagonal block: 16 float4 loads per thread, all in flight together
    constexpr int NV = NB * NB / 4 / 256;
    float4 v[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int e = t + 256 * k;
      v[k] = *reinterpret_cast<const float4*>(base + (e >> 5) * n + (e & 31) * 4);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int e = t + 256 * k;
      *reinterpret_cast<float4*>(As + (e >> 5) * LS + (e & 31) * 4) = v[k];
    }
  }
  for (int e = t; e < NB * LS; e += 256) Xs[e] = 0.f;
  __syncthreads();

  // ---- Cholesky and diagonal-block inverses, four panels
#pragma unroll 1
  for (int p = 0; p < 4; ++p) {
    const int C0 = 32 * p;
    if (w == 0) leaf_diag32(As, Xs, k0, info, C0);
    __syncthreads();
    if (p < 3) {
      leaf_trsm_below(As, Xs, C0);
      __syncthreads();
      leaf_syrk(As, C0, C0 + 32);
      __syncthreads();
    }
  }

  // ---- off-diagonal blocks: X_ip = -X_ii sum_{k=p}^{i-1} L_ik X_kp. Wave p
  // owns block column p (i = p+1 .. 3 in order); the sum goes through the
  // unused upper block (p, i) of Xs, zeroed again on the way out.
  if (w < 3) {
    const int p = w;
    for (int i = p + 1; i < 4; ++i) {
      f32x16 acc;
      acc_zero(acc);
      mma32<false>(As + (32 * i) * LS + 32 * p, Xs + (32 * p) * LS + 32 * p, 32 * (i - p), 1.f, acc);
      float* Tb = Xs + (32 * p) * LS + 32 * i;
      acc_store(Tb, acc);
      acc_zero(acc);
      mma32<false>(Xs + (32 * i) * LS + 32 * i, Tb, 32, -1.f, acc);
      acc_store(Xs + (32 * i) * LS + 32 * p, acc);
    }
  }
  __syncthreads();

  // ---- write L (lower, zeros above) and its inverse
  for (int e = t; e < NB * NB / 4; e += 256) {
    const int r = e >> 5, c = (e & 31) * 4;
    const float4 l = *reinterpret_cast<const float4*>(As + r * LS + c);
    const float4 x = *reinterpret_cast<const float4*>(Xs + r * LS + c);
    // zero the strictly upper part (columns c..c+3 against row r)
    const float4 lo = make_float4(c > r ? 0.f : l.x, c + 1 > r ? 0.f : l.y, c + 2 > r ? 0.f : l.z,
                                  c + 3 > r ? 0.f : l.w);
    const float4 xo = make_float4(c > r ? 0.f : x.x, c + 1 > r ? 0.f : x.y, c + 2 > r ? 0.f : x.z,
                                  c + 3 > r ? 0.f : x.w);
    *reinterpret_cast<float4*>(base + r * n + c) = lo;
    *reinterpret_cast<float4*>(Dinv + r * NB + c) = xo;
  }
}

constexpr size_t LEAF_LDS = sizeof(float) * (size_t(NB) * LS * 2);

// Copy the inverted diagonal blocks into place (block b at (b*NB, b*NB)).
__global__ void place_diag_kernel(const float* __restrict__ Dinv, int64_t nblk, float* A,
                                  int64_t n) {
  const int64_t b = blockIdx.y;
  const int64_t r = blockIdx.x;
  const int c = threadIdx.x;
  A[(b * NB + r) * n + b * NB + c] = Dinv[b * NB * NB + r * NB + c];
}

// In-place reversal: U[n-1-i][n-1-j] = X[i][j] for i >= j, zeros below.
__global__ void reverse_out_kernel(float* A, int64_t n) {
  const int64_t i = blockIdx.y;
  for (int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; j <= i;
       j += int64_t(gridDim.x) * blockDim.x) {
    const int64_t ii = n - 1 - i, jj = n - 1 - j;
    if (i == j) {
      if (i < ii) {  // swap the diagonal pair once
        const float a = A[i * n + i];
        const float b = A[ii * n + ii];
        A[i * n + i] = b;
        A[ii * n + ii] = a;
      }
    } else {
      const float v = A[i * n + j];
      A[ii * n + jj] = v;
      A[i * n + j] = 0.f;
    }
  }
}

__global__ void set_int_kernel(int* p, int v) { *p = v; }

// Invert the lower-triangular L (ld n) in place, its NB x NB diagonal blocks
// already inverted: bottom-up doubling. Before the level of size sz, every
// aligned block [k sz, (k+1) sz) and the trailing block [floor(n/sz) sz, n)
// are inverted; adjacent pairs (A, C) are merged with
//   X21 = -X22 (L21 X11),
// all equal-size pairs of a level in one batched GEMM each.
kq_status trtri_levels(float* L, int64_t n, float* T, hipStream_t s) {
  for (int64_t sz = NB; sz < n; sz *= 2) {
    const int64_t pair = 2 * sz;
    const int64_t nfull = n / pair;
    if (nfull > 0) {
      GemmArgs g1 = gemm_args(L + sz * n, n, L, n, T, sz, sz, sz, sz, 1.f, 0.f, G_B_LOWER);
      g1.batch = int(nfull);
      g1.strideA = pair * n + pair;
      g1.strideB = pair * n + pair;
      g1.strideC = sz * sz;
      KQ_TRY(gemm_f32(g1, s));
      GemmArgs g2 = gemm_args(L + sz * n + sz, n, T, sz, L + sz * n, n, sz, sz, sz, -1.f, 0.f,
                              G_A_LOWER | G_ORDER_MDESC);
      g2.Cin = nullptr;
      g2.batch = int(nfull);
      g2.strideA = pair * (n + 1);
      g2.strideB = sz * sz;
      g2.strideC = pair * (n + 1);
      KQ_TRY(gemm_f32(g2, s));
    }
    const int64_t r = nfull * pair;
    const int64_t rest = n - r;
    if (rest > sz) {
      const int64_t s2 = rest - sz;
      float* X11 = L + r * n + r;
      float* L21 = L + (r + sz) * n + r;
      float* X22 = L + (r + sz) * n + r + sz;
      KQ_TRY(gemm_f32(gemm_args(L21, n, X11, n, T, sz, s2, sz, sz, 1.f, 0.f, G_B_LOWER), s));
      GemmArgs g2 = gemm_args(X22, n, T, sz, L21, n, s2, sz, s2, -1.f, 0.f, G_A_LOWER | G_ORDER_MDESC);
      g2.Cin = nullptr;
      KQ_TRY(gemm_f32(g2, s));
    }
  }
  return KQ_OK;
}

}  // namespace

size_t chol_ws_bytes(int64_t n) {
  Arena ar{nullptr, 0, 0};
  ar.take<float>(size_t(n) * NB);               // inverted diagonal blocks
  ar.take<float>(size_t(n) * n / 4 + 4);        // triangular-inverse temporary
  ar.take<double>(1);
  ar.take<int>(1);
  return ar.used;
}

kq_status chol_inv_run(const float* H, int64_t n, float damp, float* U, int32_t* info,
                       Arena& ws, hipStream_t s) {
  const int64_t nb = n / NB;
  float* Dinv = ws.take<float>(size_t(n) * NB);
  float* T = ws.take<float>(size_t(n) * n / 4 + 4);
  double* dsum = ws.take<double>(1);
  int* dinfo = ws.take<int>(1);
  if (!Dinv || !T || !dsum || !dinfo) return fail(KQ_ERR_WORKSPACE, "cholesky_inv: workspace too small");

  set_int_kernel<<<1, 1, 0, s>>>(dinfo, INT_MAX);
  KQ_HIP(hipGetLastError());
  KQ_TRY(diag_sum(H, n, dsum, s));
  reverse_damp_kernel<<<dim3(unsigned(cdiv(n, 256)), unsigned(n)), 256, 0, s>>>(H, n, dsum, damp, U);
  KQ_HIP(hipGetLastError());

  KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(leaf_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(LEAF_LDS)));
  float* A = U;
  for (int64_t k = 0; k < nb; ++k) {
    const int64_t k0 = k * NB;
    leaf_kernel<<<1, 256, LEAF_LDS, s>>>(A, n, k0, Dinv + k * NB * NB, dinfo);
    KQ_HIP(hipGetLastError());
    const int64_t m = n - k0 - NB;
    if (m <= 0) break;
    float* panel = A + (k0 + NB) * n + k0;
    // L21 = panel * Dinv_k^T into the (still unused) inverse temporary, m x NB
    // dense: out of place, so the product takes narrow tiles across N
    GemmArgs gt = gemm_args(panel, n, Dinv + k * NB * NB, NB, T, NB, m, NB, NB, 1.f, 0.f, G_TRANS_B);
    KQ_TRY(gemm_f32(gt, s));
    // trailing lower triangle -= L21 L21^T, then L21 back into place
    float* trail = A + (k0 + NB) * n + (k0 + NB);
    GemmArgs gs = gemm_args(T, NB, T, NB, trail, n, m, m, NB, -1.f, 1.f, G_TRANS_B | G_OUT_LOWER);
    KQ_TRY(gemm_f32(gs, s));
    KQ_HIP(hipMemcpy2DAsync(panel, size_t(n) * sizeof(float), T, NB * sizeof(float),
                            NB * sizeof(float), size_t(m), hipMemcpyDeviceToDevice, s));
  }

  // invert L in place
  place_diag_kernel<<<dim3(NB, unsigned(nb)), NB, 0, s>>>(Dinv, nb, A, n);
  KQ_HIP(hipGetLastError());
  KQ_TRY(trtri_levels(A, n, T, s));
  reverse_out_kernel<<<dim3(unsigned(cdiv(n, 256)), unsigned(n)), 256, 0, s>>>(A, n);
  KQ_HIP(hipGetLastError());

  int hinfo = INT_MAX;
  KQ_HIP(hipMemcpyAsync(&hinfo, dinfo, sizeof(int), hipMemcpyDeviceToHost, s));
  KQ_HIP(hipStreamSynchronize(s));
  int32_t out = 0;
  if (hinfo != INT_MAX) {
    // reversed index k (0-based) = hinfo - 1  ->  original column n-1-k
    out = int32_t(n - (hinfo - 1));
  }
  if (info) *info = out;
  if (out) return fail(KQ_ERR_NOT_PD, "cholesky_inv: matrix is not positive definite (column %d)", out - 1);
  return KQ_OK;
}

}  // namespace kq
