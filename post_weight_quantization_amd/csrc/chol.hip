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
//      panel below is solved as a GEMM with that inverse, and the trailing
//      lower triangle takes a rank-128 MFMA update;
//   3. inverts L in place by recursive halving
//      inv([[A,0],[B,C]]) = [[A^-1, 0], [-C^-1 B A^-1, C^-1]], whose two
//      GEMMs per level are triangle-aware fp32 MFMA products;
//   4. reverses indices in place to obtain U (upper, zeros below).
// A non-positive (or NaN) pivot is reported through `info`.
#include "kq_internal.h"

#include <climits>

namespace kq {

namespace {

constexpr int NB = 128;
constexpr int LP = NB + 1;  // padded LDS row

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

// Factor the NB x NB diagonal block at (k0, k0) of A (ld n) in place and
// write its inverse to Dinv (NB x NB, zeros above the diagonal).
// Thread (bi, bj) = (t / 16, t % 16) keeps the 8 x 8 sub-block (bi, bj) in
// registers; column j is published through LDS each step.
__global__ __launch_bounds__(256) void leaf_kernel(float* A, int64_t n, int64_t k0, float* Dinv,
                                                   int* info) {
  __shared__ float colbuf[NB];
  __shared__ float piv[1];
  __shared__ float Ls[NB * LP];
  const int t = threadIdx.x;
  const int bi = t >> 4, bj = t & 15;
  const bool act = bi >= bj;
  float a[8][8];
  float* base = A + k0 * n + k0;
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) a[r][c] = act ? base[(8 * bi + r) * n + 8 * bj + c] : 0.f;
  if (t < NB) colbuf[t] = 0.f;
  __syncthreads();

  // ---- Cholesky: A = L L^T
  for (int jb = 0; jb < 16; ++jb) {
#pragma unroll
    for (int jc = 0; jc < 8; ++jc) {
      const int j = 8 * jb + jc;
      if (bi == jb && bj == jb) {
        float p = a[jc][jc];
        if (!(p > 0.f)) {  // non-positive or NaN pivot
          atomicMin(info, int(k0 + j) + 1);
          p = 1.f;
        }
        const float d = sqrtf(p);
        a[jc][jc] = d;
        piv[0] = 1.f / d;
      }
      __syncthreads();
      if (bj == jb && act) {
        const float rinv = piv[0];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const bool below = (bi > jb) || (r > jc);
          if (below) a[r][jc] *= rinv;
          colbuf[8 * bi + r] = below ? a[r][jc] : 0.f;
        }
      }
      __syncthreads();
      if (act && (8 * bi + 7 > j) && (8 * bj + 7 > j)) {
        float cr[8], cc[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) cr[r] = colbuf[8 * bi + r];
#pragma unroll
        for (int c = 0; c < 8; ++c) cc[c] = colbuf[8 * bj + c];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) a[r][c] -= cr[r] * cc[c];
      }
    }
  }
  // write L (zeros above the diagonal) to A and to LDS
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int row = 8 * bi + r, col = 8 * bj + c;
      const float v = (act && col <= row) ? a[r][c] : 0.f;
      if (act) base[row * n + col] = v;
      Ls[row * LP + col] = v;
    }
  __syncthreads();

  // ---- inverse: X = L^-1 by forward elimination on B = I, row j final at step j
  float bm[8][8];
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) bm[r][c] = (bi == bj && r == c) ? 1.f : 0.f;
  __shared__ float rowbuf[NB];
  if (t < NB) rowbuf[t] = 0.f;
  __syncthreads();
  for (int jb = 0; jb < 16; ++jb) {
#pragma unroll
    for (int jc = 0; jc < 8; ++jc) {
      const int j = 8 * jb + jc;
      if (bi == jb && act) {
        const float dinv = 1.f / Ls[j * LP + j];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          bm[jc][c] *= dinv;
          rowbuf[8 * bj + c] = bm[jc][c];
        }
      }
      __syncthreads();
      if (act && 8 * bi + 7 > j) {
        float cr[8], cc[8];
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int row = 8 * bi + r;
          cr[r] = row > j ? Ls[row * LP + j] : 0.f;
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) cc[c] = rowbuf[8 * bj + c];
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
          for (int c = 0; c < 8; ++c) bm[r][c] -= cr[r] * cc[c];
      }
      __syncthreads();
    }
  }
#pragma unroll
  for (int r = 0; r < 8; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int row = 8 * bi + r, col = 8 * bj + c;
      Dinv[row * NB + col] = (act && col <= row) ? bm[r][c] : 0.f;
    }
}

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

// L (ld n) holds inverted diagonal blocks; invert the block range [b0, b0+nb).
kq_status trtri_rec(float* L, int64_t n, int64_t b0, int64_t nb, float* T, hipStream_t s) {
  if (nb <= 1) return KQ_OK;
  const int64_t n1 = (nb + 1) / 2, n2 = nb - n1;
  KQ_TRY(trtri_rec(L, n, b0, n1, T, s));
  KQ_TRY(trtri_rec(L, n, b0 + n1, n2, T, s));
  const int64_t r1 = b0 * NB, r2 = (b0 + n1) * NB;
  const int64_t m1 = n1 * NB, m2 = n2 * NB;
  float* X11 = L + r1 * n + r1;
  float* L21 = L + r2 * n + r1;
  float* X22 = L + r2 * n + r2;
  // T = L21 X11   (X11 lower: op(B)[k][c] = 0 for k < c)
  GemmArgs g1 = gemm_args(L21, n, X11, n, T, m1, m2, m1, m1, 1.f, 0.f, G_B_LOWER);
  KQ_TRY(gemm_f32(g1, s));
  // X21 = -X22 T  (X22 lower: op(A)[r][k] = 0 for k > r)
  GemmArgs g2 = gemm_args(X22, n, T, m1, L21, n, m2, m1, m2, -1.f, 0.f, G_A_LOWER);
  KQ_TRY(gemm_f32(g2, s));
  return KQ_OK;
}

}  // namespace

size_t chol_ws_bytes(int64_t n) {
  Arena ar{nullptr, 0, 0};
  ar.take<float>(size_t(n) * NB);               // inverted diagonal blocks
  const int64_t nb = cdiv(n, NB);
  const int64_t n1 = (nb + 1) / 2;
  ar.take<float>(size_t(n1 * NB) * (nb - n1) * NB + 4);  // recursion temporary
  ar.take<double>(1);
  ar.take<int>(1);
  return ar.used;
}

kq_status chol_inv_run(const float* H, int64_t n, float damp, float* U, int32_t* info,
                       Arena& ws, hipStream_t s) {
  const int64_t nb = n / NB;
  float* Dinv = ws.take<float>(size_t(n) * NB);
  const int64_t n1 = (nb + 1) / 2;
  float* T = ws.take<float>(size_t(n1 * NB) * (nb - n1) * NB + 4);
  double* dsum = ws.take<double>(1);
  int* dinfo = ws.take<int>(1);
  if (!Dinv || !T || !dsum || !dinfo) return fail(KQ_ERR_WORKSPACE, "cholesky_inv: workspace too small");

  set_int_kernel<<<1, 1, 0, s>>>(dinfo, INT_MAX);
  KQ_HIP(hipGetLastError());
  KQ_TRY(diag_sum(H, n, dsum, s));
  reverse_damp_kernel<<<dim3(unsigned(cdiv(n, 256)), unsigned(n)), 256, 0, s>>>(H, n, dsum, damp, U);
  KQ_HIP(hipGetLastError());

  float* A = U;
  for (int64_t k = 0; k < nb; ++k) {
    const int64_t k0 = k * NB;
    leaf_kernel<<<1, 256, 0, s>>>(A, n, k0, Dinv + k * NB * NB, dinfo);
    KQ_HIP(hipGetLastError());
    const int64_t m = n - k0 - NB;
    if (m <= 0) break;
    float* panel = A + (k0 + NB) * n + k0;
    // panel <- panel * Dinv_k^T   (in place: each tile reads its rows before writing them)
    GemmArgs gt = gemm_args(panel, n, Dinv + k * NB * NB, NB, panel, n, m, NB, NB, 1.f, 0.f, G_TRANS_B);
    KQ_TRY(gemm_f32(gt, s));
    // trailing lower triangle -= panel panel^T
    float* trail = A + (k0 + NB) * n + (k0 + NB);
    GemmArgs gs = gemm_args(panel, n, panel, n, trail, n, m, m, NB, -1.f, 1.f, G_TRANS_B | G_OUT_LOWER);
    KQ_TRY(gemm_f32(gs, s));
  }

  // invert L in place
  place_diag_kernel<<<dim3(NB, unsigned(nb)), NB, 0, s>>>(Dinv, nb, A, n);
  KQ_HIP(hipGetLastError());
  KQ_TRY(trtri_rec(A, n, 0, nb, T, s));
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
