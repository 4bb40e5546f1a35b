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
//   2. factors A = L L^T in place with 128-column blocks inside 512-column
//      superblocks: a single-workgroup leaf factors the diagonal block in
//      LDS and writes only the inverse of its factor (the diagonal blocks of
//      L itself are never needed again), the panel below is solved as a GEMM
//      with that inverse into a compact copy of the superblock's panels, the
//      superblock's remaining columns take a rank-128 MFMA update from it,
//      and after each superblock the rest of the trailing lower triangle
//      takes one rank-512 update from it before one copy puts the
//      superblock's panels in place;
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

constexpr int NB = 128;   // leaf (diagonal block) size
constexpr int SB = 512;   // superblock: columns between two full trailing updates

// A[i][j] = H[n-1-i][n-1-j] + delta [i == j] for i >= j (reads H's upper triangle)
// A[i][j] = H[n-1-i][n-1-j] (+ delta on the diagonal) for j <= i, four
// columns per thread: the float4 at H[n-1-i][n-4-j ..] reversed lands at
// A[i][j ..]; columns past the diagonal are left alone. n % 4 == 0. Grid:
// (column quads / 256, n).
__global__ void reverse_damp_kernel(const float* __restrict__ H, int64_t n, const double* dsum,
                                    float damp, float* __restrict__ A) {
  const int64_t i = blockIdx.y;
  const int64_t j = 4 * (int64_t(blockIdx.x) * blockDim.x + threadIdx.x);
  if (j > i) return;
  const float delta = float(double(damp) * (*dsum) / double(n));
  const float4 h = *reinterpret_cast<const float4*>(H + (n - 1 - i) * n + (n - 4 - j));
  float v[4] = {h.w, h.z, h.y, h.x};
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] += j + q == i ? delta : 0.f;
  if (j + 3 <= i) {
    *reinterpret_cast<float4*>(A + i * n + j) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (j + q <= i) A[i * n + j + q] = v[q];
  }
}

// ---------------------------------------------------------------- the leaf
// Factor the NB x NB diagonal block at (k0, k0) of A (ld n) in LDS and write
// the inverse of its factor to Dinv (NB x NB, zeros above the diagonal). The
// factor itself is not written back: only its inverse is used afterwards
// (for the panel solve and as the diagonal blocks of the inverse). One
// workgroup of 4 waves. Right-looking over eight 16-column panels p:
//  * wave 0 factors the panel's 16 x 16 diagonal block in registers (DPP
//    row broadcasts, no LDS access inside the 16 column steps) and keeps the
//    reciprocals of its diagonal;
//  * the rows below solve for the panel's columns by forward substitution,
//    one row per thread, while wave 2 inverts the panel's diagonal block
//    (one column per thread);
//  * wave 0 applies the panel to the next diagonal block and factors it
//    right away; waves 1..3 bring the next block column below the diagonal
//    up to date in one product over all panels so far (left-looking) and
//    apply the panel to the later diagonal blocks, all in 16 x 16 blocks on
//    the matrix cores (v_mfma_f32_16x16x4f32).
// The blocks of the inverse X = L^-1 below the diagonal follow by doubling,
// X21 = -X22 (L21 X11) over 16 -> 32 -> 64 -> 128, on the matrix cores.
constexpr int LS = NB + 4;  // LDS row stride (floats), keeps float4 alignment
constexpr int PW = 16;      // panel width
constexpr int NP = NB / PW;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Broadcast of lane J of each 16-lane row (DPP row_newbcast) to that row.
template <int J>
__device__ inline float bc16(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + J,
                                                            0xF, 0xF, true));
}

// x[J + 1 + K] += nl * L[J + 1 + K][J] (lane J + 1 + K's x[J]), nl = -L[r][J]
template <int J, int... K>
__device__ inline void fac16_upd(float (&x)[16], float nl, std::integer_sequence<int, K...>) {
  ((x[J + 1 + K] = __builtin_fmaf(bc16<J + 1 + K>(x[J]), nl, x[J + 1 + K])), ...);
}

// Column J of the 16 x 16 Cholesky factor: the pivot is lane J's x[J];
// every row scales its x[J] by the pivot's reciprocal square root (row J
// gets sqrt(pivot)), then the columns right of J take the rank-1 update.
// Only the lower triangle of the block is ever read; a non-positive (or
// NaN) pivot is kept in dv for the caller and replaced by 1.
template <int J>
struct Fac16 {
  __device__ static void run(float (&x)[16], float (&dv)[16], float (&rv)[16]) {
    const float piv = bc16<J>(x[J]);
    dv[J] = piv;
    const float rs = __builtin_amdgcn_rsqf(piv > 0.f ? piv : 1.f);
    rv[J] = rs;
    x[J] *= rs;
    fac16_upd<J>(x, -x[J], std::make_integer_sequence<int, 15 - J>{});
    Fac16<J + 1>::run(x, dv, rv);
  }
};
template <>
struct Fac16<16> {
  __device__ static void run(float (&)[16], float (&)[16], float (&)[16]) {}
};

// Cholesky factor of the 16 x 16 block at (R0, R0) of As (row stride LS),
// in place (its upper triangle left undefined), by one wave: lane r % 16
// holds row r (the four 16-lane rows hold copies). The reciprocals of the
// factor's diagonal go to invd[R0 ..]; the first bad pivot to info.
__device__ inline void fac16_block(float* As, float* invd, int R0, int col0, int* info) {
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  float x[16], dv[16], rv[16];
  float* row = As + (R0 + r) * LS + R0;
#pragma unroll
  for (int k = 0; k < 16; k += 4) {
    const float4 v = *reinterpret_cast<const float4*>(row + k);
    x[k] = v.x;
    x[k + 1] = v.y;
    x[k + 2] = v.z;
    x[k + 3] = v.w;
  }
  Fac16<0>::run(x, dv, rv);
  if (lane < 16) {
#pragma unroll
    for (int k = 0; k < 16; k += 4)
      *reinterpret_cast<float4*>(row + k) = make_float4(x[k], x[k + 1], x[k + 2], x[k + 3]);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 16; k += 4)
      *reinterpret_cast<float4*>(invd + R0 + k) = make_float4(rv[k], rv[k + 1], rv[k + 2], rv[k + 3]);
    for (int k = 0; k < 16; ++k)
      if (!(dv[k] > 0.f)) {
        atomicMin(info, col0 + k + 1);
        break;
      }
  }
}

// Rows 0..15 of a 16 x 16 lower block at (P0, P0) of As into registers
// (l[c][m] for m < c, broadcast reads, all in flight together) and the
// reciprocals of its diagonal.
__device__ inline void load_diag16(const float* As, const float* invd, int P0, float (&l)[PW][PW],
                                   float (&iv)[PW]) {
#pragma unroll
  for (int c = 0; c < PW; ++c)
#pragma unroll
    for (int m = 0; m < PW; m += 4) {
      if (m < c) {
        const float4 v = *reinterpret_cast<const float4*>(As + (P0 + c) * LS + P0 + m);
        l[c][m] = v.x;
        l[c][m + 1] = v.y;
        l[c][m + 2] = v.z;
        l[c][m + 3] = v.w;
      }
    }
#pragma unroll
  for (int m = 0; m < PW; m += 4) {
    const float4 v = *reinterpret_cast<const float4*>(invd + P0 + m);
    iv[m] = v.x;
    iv[m + 1] = v.y;
    iv[m + 2] = v.z;
    iv[m + 3] = v.w;
  }
}

// Column c of the inverse of the 16 x 16 lower block at (P0, P0): L x = e_c
// by forward substitution, into Xs.
__device__ inline void inv16_col(const float* As, const float* invd, float* Xs, int P0, int c) {
  float l[PW][PW], iv[PW], x[PW];
  load_diag16(As, invd, P0, l, iv);
  // right-looking: once x[r] is final it updates every later entry, so the
  // dependent chain is one multiply and one FMA per row
#pragma unroll
  for (int r = 0; r < PW; ++r) x[r] = r == c ? 1.f : 0.f;
#pragma unroll
  for (int r = 0; r < PW; ++r) {
    x[r] *= iv[r];
#pragma unroll
    for (int m = r + 1; m < PW; ++m) x[m] = __builtin_fmaf(-l[m][r], x[r], x[m]);
  }
#pragma unroll
  for (int r = 0; r < PW; ++r) Xs[(P0 + r) * LS + P0 + c] = x[r];
}

// Lane l supplies A[l % 16][k + l / 16] and B(k + l / 16, l % 16) to
// v_mfma_f32_16x16x4f32; element r of its accumulator is
// C[4 (l / 16) + r][l % 16].
template <bool TB>
__device__ inline void chunk16(const float* Ap, const float* Bp, int k0, float (&a)[4], float (&b)[4]) {
  const int lane = threadIdx.x & 63;
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = k0 + 4 * q + lk;
    a[q] = Ap[li * LS + k];
    b[q] = TB ? Bp[li * LS + k] : Bp[k * LS + li];
  }
}

// C (16 x 16, rows/cols given by pointers with stride LS) += sgn * A B^T
// over K = kn (a multiple of 16):
//   A[i][k] = Ap[i * LS + k], B[j][k] = Bp[j * LS + k] (TB) or Bp[k * LS + j].
// The next 16-deep chunk is read while the current one's MFMAs run.
template <bool TB>
__device__ inline void mma16(const float* Ap, const float* Bp, int kn, float sgn, f32x4& acc) {
  float a[4], b[4];
  chunk16<TB>(Ap, Bp, 0, a, b);
  for (int k0 = 0; k0 < kn; k0 += 16) {
    float an[4], bn[4];
    chunk16<TB>(Ap, Bp, k0 + 16 < kn ? k0 + 16 : k0, an, bn);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(sgn * a[q], b[q], acc, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = an[q];
      b[q] = bn[q];
    }
  }
}

__device__ inline void acc16_load(const float* C, f32x4& acc) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = C[(4 * (lane >> 4) + r) * LS + (lane & 15)];
}

__device__ inline void acc16_store(float* C, const f32x4& acc) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < 4; ++r) C[(4 * (lane >> 4) + r) * LS + (lane & 15)] = acc[r];
}

__device__ inline void wave_lds_fence() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// C_b -= P_bi P_bj^T for one block (K = 16)
__device__ inline void syrk16_one(float* As, int R0, int C0, int bi, int bj) {
  float* Cp = As + (R0 + PW * bi) * LS + R0 + PW * bj;
  f32x4 acc;
  acc16_load(Cp, acc);
  float a[4], b[4];
  chunk16<true>(As + (R0 + PW * bi) * LS + C0, As + (R0 + PW * bj) * LS + C0, 0, a, b);
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(-a[q], b[q], acc, 0, 0, 0);
  acc16_store(Cp, acc);
}

__global__ __launch_bounds__(256) void leaf_kernel(const float* A, int64_t n, int64_t k0,
                                                   float* Dinv, int* info) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* As = sm;                    // NB x LS: the block, then L
  float* Xs = sm + NB * LS;          // NB x LS: the inverse (upper blocks: scratch)
  float* invd = Xs + NB * LS;        // NB: reciprocals of L's diagonal
  const int t = threadIdx.x;
  const int w = t >> 6;
  {
    // the diagonal block: 16 float4 loads per thread, all in flight together
    const float* base = A + k0 * n + k0;
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
  __syncthreads();
  if (w == 0) fac16_block(As, invd, 0, int(k0), info);
  __syncthreads();

#pragma unroll 1
  for (int p = 0; p + 1 < NP; ++p) {
    const int C0 = PW * p;
    const int R0 = C0 + PW;   // first row (and column) below the panel
    const int R = NB - R0;    // rows below
    // ---- forward substitution: L[r][C0 + c] L[C0 + c][C0 + c] =
    //      A[r][C0 + c] - sum_{m < c} L[r][C0 + m] L[C0 + c][C0 + m],
    //      each term subtracted as soon as L[r][C0 + m] is known
    if (t < R) {
      const int r = R0 + t;
      float a[PW], l[PW][PW], iv[PW];
      float* arow = As + r * LS + C0;
#pragma unroll
      for (int c = 0; c < PW; c += 4) {
        const float4 v = *reinterpret_cast<const float4*>(arow + c);
        a[c] = v.x;
        a[c + 1] = v.y;
        a[c + 2] = v.z;
        a[c + 3] = v.w;
      }
      load_diag16(As, invd, C0, l, iv);
      // right-looking: a[c] final, then it updates every later column
#pragma unroll
      for (int c = 0; c < PW; ++c) {
        a[c] *= iv[c];
#pragma unroll
        for (int m = c + 1; m < PW; ++m) a[m] = __builtin_fmaf(-a[c], l[m][c], a[m]);
      }
#pragma unroll
      for (int c = 0; c < PW; c += 4)
        *reinterpret_cast<float4*>(arow + c) = make_float4(a[c], a[c + 1], a[c + 2], a[c + 3]);
    } else if (t >= 128 && t < 128 + PW) {
      inv16_col(As, invd, Xs, C0, t - 128);
    }
    __syncthreads();
    // ---- updates. Wave 0 applies the panel to the next diagonal block and
    // factors it. Waves 1..3 bring the next block column below the diagonal
    // up to date in one product over all panels so far (its blocks are
    // untouched until then: left-looking), and apply the panel to the later
    // diagonal blocks (right-looking), so each phase carries about the same
    // work instead of the whole trailing triangle at the first panels.
    if (w == 0) {
      syrk16_one(As, R0, C0, 0, 0);
      wave_lds_fence();
      fac16_block(As, invd, R0, int(k0) + R0, info);
    } else {
      const int nxt = p + 1;              // the next block column
      const int ntask = 2 * (NP - 1 - nxt);
      for (int task = w - 1; task < ntask; task += 3) {
        if (task < NP - 1 - nxt) {
          // block (i, nxt) -= sum over panels 0..p of L_i,c L_nxt,c^T
          const int i = nxt + 1 + task;
          float* Cb = As + (PW * i) * LS + PW * nxt;
          f32x4 acc;
          acc16_load(Cb, acc);
          mma16<true>(As + (PW * i) * LS, As + (PW * nxt) * LS, PW * nxt, -1.f, acc);
          acc16_store(Cb, acc);
        } else {
          // diagonal block (j, j) -= L_j,p L_j,p^T
          const int j = nxt + 1 + (task - (NP - 1 - nxt));
          syrk16_one(As, R0, C0, j - nxt, j - nxt);
        }
      }
    }
    __syncthreads();
  }
  // the last panel's diagonal block
  if (t < PW) inv16_col(As, invd, Xs, NB - PW, t);
  __syncthreads();

  // ---- the blocks of the inverse below the diagonal, by doubling: merge
  // adjacent inverted blocks with X21 = -X22 (L21 X11), 16 -> 32 -> 64 -> 128.
  // In a merge the product T = L21 X11 goes to an unused upper part of Xs
  // (rows of the first half, columns of the second: each block column of T
  // a k-major slab). In the first two levels the wave that computes T's
  // column b also computes X21's column b from it; the last level splits T
  // by rows and X21 by columns, with a barrier between.
  {
    // level 1: wave w merges blocks 2w and 2w + 1
    const int a0 = 2 * w;
    f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
    mma16<false>(As + (PW * (a0 + 1)) * LS + PW * a0, Xs + (PW * a0) * LS + PW * a0, PW, 1.f, tacc);
    float* Tb = Xs + (PW * a0) * LS + PW * (a0 + 1);
    acc16_store(Tb, tacc);
    wave_lds_fence();
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    mma16<false>(Xs + (PW * (a0 + 1)) * LS + PW * (a0 + 1), Tb, PW, -1.f, o);
    acc16_store(Xs + (PW * (a0 + 1)) * LS + PW * a0, o);
  }
  __syncthreads();
  {
    // level 2: merge q = w / 2 joins blocks {4q, 4q+1} and {4q+2, 4q+3};
    // this wave takes block column b = w % 2 of T and of X21
    const int q0 = 4 * (w >> 1), b = w & 1, c0 = q0 + 2;
    float* slab = Xs + (PW * q0) * LS + PW * (c0 + b);  // T[c][b] at block (q0 + c, c0 + b)
#pragma unroll 1
    for (int a = 0; a < 2; ++a) {
      f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
      mma16<false>(As + (PW * (c0 + a)) * LS + PW * (q0 + b), Xs + (PW * (q0 + b)) * LS + PW * (q0 + b),
                   PW * (2 - b), 1.f, tacc);
      acc16_store(slab + (PW * a) * LS, tacc);
    }
    wave_lds_fence();
#pragma unroll 1
    for (int a = 0; a < 2; ++a) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      mma16<false>(Xs + (PW * (c0 + a)) * LS + PW * c0, slab, PW * (a + 1), -1.f, o);
      acc16_store(Xs + (PW * (c0 + a)) * LS + PW * (q0 + b), o);
    }
  }
  __syncthreads();
  {
    // level 3: blocks 0..3 and 4..7. T's blocks have K = 16 (4 - b) and
    // X21's K = 16 (a + 1), so T goes by block rows (wave a) and X21 by block
    // columns (wave b) after a barrier: ten 16-deep chunks per wave in each
    // half. T[a][b] sits at block (a, 4 + b): column b of T is a k-major slab.
    const int a = w;
#pragma unroll 1
    for (int b = 0; b < 4; ++b) {
      f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
      mma16<false>(As + (PW * (4 + a)) * LS + PW * b, Xs + (PW * b) * LS + PW * b, PW * (4 - b), 1.f, tacc);
      acc16_store(Xs + (PW * a) * LS + PW * (4 + b), tacc);
    }
  }
  __syncthreads();
  {
    const int b = w;
    const float* slab = Xs + PW * (4 + b);
#pragma unroll 1
    for (int a = 0; a < 4; ++a) {
      f32x4 o = {0.f, 0.f, 0.f, 0.f};
      mma16<false>(Xs + (PW * (4 + a)) * LS + PW * 4, slab, PW * (a + 1), -1.f, o);
      acc16_store(Xs + (PW * (4 + a)) * LS + PW * b, o);
    }
  }
  __syncthreads();

  // ---- write the inverse (zeros above the diagonal)
  for (int e = t; e < NB * NB / 4; e += 256) {
    const int r = e >> 5, c = (e & 31) * 4;
    const float4 x = *reinterpret_cast<const float4*>(Xs + r * LS + c);
    const float4 xo = make_float4(c > r ? 0.f : x.x, c + 1 > r ? 0.f : x.y, c + 2 > r ? 0.f : x.z,
                                  c + 3 > r ? 0.f : x.w);
    *reinterpret_cast<float4*>(Dinv + r * NB + c) = xo;
  }
}

constexpr size_t LEAF_LDS = sizeof(float) * (size_t(NB) * LS * 2 + NB);

// Copy the inverted diagonal blocks into place (block b at (b*NB, b*NB)).
__global__ void place_diag_kernel(const float* __restrict__ Dinv, int64_t nblk, float* A,
                                  int64_t n) {
  const int64_t b = blockIdx.y;
  const int64_t r = blockIdx.x;
  const int c = threadIdx.x;
  A[(b * NB + r) * n + b * NB + c] = Dinv[b * NB * NB + r * NB + c];
}

// In-place reversal: U[n-1-i][n-1-j] = X[i][j] for i >= j, zeros below.
// U[n-1-i][n-1-j] = A[i][j] for j < i (zeroing A[i][j]) and the diagonal
// reversed, in place, four columns per thread: A[i][j ..] (float4) goes
// reversed to A[n-1-i][n-4-j ..]. Row n-1-i's target columns lie above its
// diagonal, which no thread reads. n % 4 == 0. Grid: (column quads / 256, n).
__global__ void reverse_out_kernel(float* A, int64_t n) {
  const int64_t i = blockIdx.y;
  const int64_t j = 4 * (int64_t(blockIdx.x) * blockDim.x + threadIdx.x);
  if (j > i) return;
  const int64_t ii = n - 1 - i;
  if (j + 3 < i) {
    const float4 v = *reinterpret_cast<const float4*>(A + i * n + j);
    *reinterpret_cast<float4*>(A + ii * n + (n - 4 - j)) = make_float4(v.w, v.z, v.y, v.x);
    *reinterpret_cast<float4*>(A + i * n + j) = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  // the quad that holds the diagonal: strictly-lower entries as above, then
  // the diagonal pair swapped once (by the row with i < n-1-i)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t jq = j + q;
    if (jq < i) {
      A[ii * n + (n - 1 - jq)] = A[i * n + jq];
      A[i * n + jq] = 0.f;
    } else if (jq == i && i < ii) {
      const float a = A[i * n + i];
      const float b = A[ii * n + ii];
      A[i * n + i] = b;
      A[ii * n + ii] = a;
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
      GemmArgs g1 = gemm_args(L + sz * n, n, L, n, T, sz, sz, sz, sz, 1.f, 0.f, G_B_LOWER | G_ORDER_NASC);
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
      KQ_TRY(gemm_f32(gemm_args(L21, n, X11, n, T, sz, s2, sz, sz, 1.f, 0.f, G_B_LOWER | G_ORDER_NASC), s));
      GemmArgs g2 = gemm_args(X22, n, T, sz, L21, n, s2, sz, s2, -1.f, 0.f, G_A_LOWER | G_ORDER_MDESC);
      g2.Cin = nullptr;
      KQ_TRY(gemm_f32(g2, s));
    }
  }
  return KQ_OK;
}

}  // namespace

// The temporary holds one superblock's solved panels (rows below its first
// leaf, SB columns) during the factorization and the products of the
// triangular inverse (n^2 / 4) afterwards.
static size_t chol_tmp_floats(int64_t n) {
  const size_t panels = size_t(std::max<int64_t>(n - NB, 0)) * size_t(std::min<int64_t>(SB, n));
  return std::max(panels, size_t(n) * n / 4) + 4;
}

size_t chol_ws_bytes(int64_t n) {
  Arena ar{nullptr, 0, 0};
  ar.take<float>(size_t(n) * NB);               // inverted diagonal blocks
  ar.take<float>(chol_tmp_floats(n));          // superblock panels, then the inverse temporary
  ar.take<double>(1);
  ar.take<int>(1);
  return ar.used;
}

kq_status chol_inv_run(const float* H, int64_t n, float damp, float* U, int32_t* info,
                       Arena& ws, hipStream_t s) {
  const int64_t nb = n / NB;
  float* Dinv = ws.take<float>(size_t(n) * NB);
  float* T = ws.take<float>(chol_tmp_floats(n));
  double* dsum = ws.take<double>(1);
  int* dinfo = ws.take<int>(1);
  if (!Dinv || !T || !dsum || !dinfo) return fail(KQ_ERR_WORKSPACE, "cholesky_inv: workspace too small");

  set_int_kernel<<<1, 1, 0, s>>>(dinfo, INT_MAX);
  KQ_HIP(hipGetLastError());
  KQ_TRY(diag_sum(H, n, dsum, s));
  reverse_damp_kernel<<<dim3(unsigned(cdiv(n / 4, 256)), unsigned(n)), 256, 0, s>>>(H, n, dsum, damp, U);
  KQ_HIP(hipGetLastError());

  KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(leaf_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(LEAF_LDS)));
  // Two levels of blocking: superblocks of SB columns, each factored
  // right-looking in NB-column steps whose trailing updates stay inside the
  // superblock's columns (all rows below); after the superblock one rank-SB
  // update brings the rest of the trailing triangle up to date. The big
  // update reads and writes the trailing triangle once per SB columns
  // instead of once per NB, which keeps it compute-bound at large n.
  float* A = U;
  for (int64_t S0 = 0; S0 < n; S0 += SB) {
    const int64_t S1 = std::min<int64_t>(S0 + SB, n);
    const int64_t sw = S1 - S0;
    // TS: the superblock's solved panels, row r >= S0 + NB of column c in
    // [S0, S1) at TS[(r - S0 - NB) sw + (c - S0)]
    float* TS = T;
    for (int64_t k0 = S0; k0 < S1; k0 += NB) {
      const int64_t k = k0 / NB;
      leaf_kernel<<<1, 256, LEAF_LDS, s>>>(A, n, k0, Dinv + k * NB * NB, dinfo);
      KQ_HIP(hipGetLastError());
      const int64_t m = n - k0 - NB;  // rows below the block
      if (m <= 0) break;
      const float* panel = A + (k0 + NB) * n + k0;
      float* Tk = TS + (k0 - S0) * sw + (k0 - S0);
      // L21 = panel * Dinv_k^T (Dinv_k lower: op(B)[k][j] = 0 for k > j),
      // out of place into TS, so the product takes narrow tiles across N
      GemmArgs gt = gemm_args(panel, n, Dinv + k * NB * NB, NB, Tk, sw, m, NB, NB, 1.f, 0.f,
                              G_TRANS_B | G_B_UPPER);
      KQ_TRY(gemm_f32(gt, s));
      // the superblock's remaining columns (all rows below) -= L21 L21^T
      const int64_t w = S1 - k0 - NB;
      if (w > 0) {
        float* trail = A + (k0 + NB) * n + (k0 + NB);
        GemmArgs gs = gemm_args(Tk, sw, Tk, sw, trail, n, m, w, NB, -1.f, 1.f, G_TRANS_B | G_OUT_LOWER);
        KQ_TRY(gemm_f32(gs, s));
      }
    }
    const int64_t rows = n - S0 - NB;
    if (rows <= 0) continue;
    // the rest of the trailing lower triangle -= L_S L_S^T, L_S = TS rows from S1
    const int64_t mt = n - S1;
    if (mt > 0) {
      const float* LS = TS + (S1 - S0 - NB) * sw;
      float* trail = A + S1 * n + S1;
      GemmArgs gb = gemm_args(LS, sw, LS, sw, trail, n, mt, mt, sw, -1.f, 1.f, G_TRANS_B | G_OUT_LOWER);
      KQ_TRY(gemm_f32(gb, s));
    }
    // the panels back into place in one copy: the entries of TS above each
    // panel were never written and land in the diagonal blocks or the upper
    // triangle, which the inverse overwrites and never reads
    KQ_HIP(hipMemcpy2DAsync(A + (S0 + NB) * n + S0, size_t(n) * sizeof(float), TS, size_t(sw) * sizeof(float),
                            size_t(sw) * sizeof(float), size_t(rows), hipMemcpyDeviceToDevice, s));
  }

  // The pivot status is final once the last leaf has run. Reading it here,
  // before the inverse is enqueued, leaves the inverse and the index reversal
  // (about a fifth of the stage) queued when the call returns, so the
  // caller's next launches reach the stream before it drains.
  int hinfo = INT_MAX;
  KQ_TRY(read_to_host(&hinfo, dinfo, sizeof(int), s));
  int32_t out = 0;
  if (hinfo != INT_MAX) {
    // reversed index k (0-based) = hinfo - 1  ->  original column n-1-k
    out = int32_t(n - (hinfo - 1));
  }
  if (info) *info = out;
  if (out) return fail(KQ_ERR_NOT_PD, "cholesky_inv: matrix is not positive definite (column %d)", out - 1);

  // invert L in place
  place_diag_kernel<<<dim3(NB, unsigned(nb)), NB, 0, s>>>(Dinv, nb, A, n);
  KQ_HIP(hipGetLastError());
  KQ_TRY(trtri_levels(A, n, T, s));
  reverse_out_kernel<<<dim3(unsigned(cdiv(n / 4, 256)), unsigned(n)), 256, 0, s>>>(A, n);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

}  // namespace kq
