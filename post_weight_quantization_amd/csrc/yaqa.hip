// Rounding with output-side feedback: the generalized LDLQ of YAQA on
// KronQ's Kronecker sketch H_G' (x) H_X'.
//
// Notes on YAQA (arXiv 2505.22988), section "key designs", item 4: for a
// sketch H_O (x) H_I with unit-triangular LDL factors L_O, L_I the rounding
// is the fixed point of W = Q(W* + L_O'^T Dl L_I' + L_O'^T Dl + Dl L_I'),
// Dl = W* - W, L' = L - I; item 1: it settles within m + n - 1 steps because
// entry (i, j) is fed back only from entries above-left of it. With the
// inverse factors of both sides (upper U, U^T U = H^-1, from kq_cholesky_inv)
// the fed-back input of entry (i, j) is
//   z_ij = W*_ij - sum_{k<=i, l<=j, (k,l)!=(i,j)} U_O[k,i] e_kl U_I[l,j],
//   e_kl = (z_kl - w^_kl) / (U_O[k,k] U_I[l,l]),
// the KronQ sweep's GPTQ update along each row plus the same update along
// each column. Every order that visits (k,l) before (i,j) whenever k <= i and
// l <= j gives the same codes.
//
// Order used here: a wavefront over 64 x 64 tiles. The tiles (I, J) with
// I + J = s form one launch, one workgroup per tile, and inside a tile the
// entries run as a skewed wavefront (row i reaches column j at step 2 i + j,
// below).
// What a tile needs from outside arrives through two accumulators in HBM:
//   M[I,J] = sum_{L<=J} e_{I,L} U_I[L,J]            (row feedback)
//   Wk     = W* - sum_{K<I} U_O[K,I]^T M[K,J]          (column feedback)
// A tile starts from Z0 = Wk_IJ - U_O[I,I]^T Mpart_IJ, Mpart holding the
// column blocks L < J. The feedback of its two neighbours finished one step
// earlier (left: e_{I,J-1} U_I[J-1,J]; above: U_O[I-1,I]^T M_{I-1,J}) the tile
// computes itself as MFMA products in LDS; everything farther away arrives
// through 64 x 64 x 64 fp32 MFMA products that carry the results of step s to
// the tiles of steps >= s + 2:
// M[I, blocks >= J+2] += e_IJ U_I[J, .] and Wk[blocks >= I+2, J] -= U_O[I, .]^T M_IJ.
// They run in the launch of step s + 1, on the workgroups after its tiles
// (the CUs the tiles leave free), so one launch per step carries all of it.
//
// Inside a tile, the four lanes of a quad hold one row (16 columns each) as
// v = Z0 - (column feedback received) and t = sum_{l<j} e_il U_I[l,j], so
// z = v - U_O[i,i] t. Row i reaches column j at step 2 i + j: the rounded
// front entry's e goes along its row (t += e U_I[j, :]) by DPP within the
// quad, and its T = t + (z - w^) / U_O[i,i] (= sum_{l<=j} e_il U_I[l,j]) down
// its column (v -= U_O[i, r] T for rows r below) through LDS, read after the
// step's barrier and applied one step later, before the row below needs it.
#include "kq_internal.h"

#include <algorithm>

namespace kq {

namespace {

constexpr int YT = 64;            // tile
constexpr int YSEG = 16;          // columns per thread
constexpr int YNSEG = YT / YSEG;  // threads per tile row
constexpr int YP = YT + 4;        // padded LDS row (floats)
constexpr int YCP = YT + 16;      // padded code row (bytes)

static_assert(YNSEG * YT == 256, "one tile row per YNSEG threads, 256 threads");

constexpr size_t YAQA_LDS = sizeof(float) * (8 * YT * YP + YT + 4 * YT) + YT * YCP;

typedef float f32x16 __attribute__((ext_vector_type(16)));

struct YaqaStep {
  float* Wk;        // m_p x n_p working input (column feedback applied)
  float* Mp;        // m_p x n_p row-feedback accumulator; a finished tile holds its complete M
  float* E;         // m_p x n_p scaled errors
  int64_t ld;       // n_p
  const float* UI;  // n_p x n_p (row stride ldI)
  const float* UO;  // m_p x m_p (row stride ldO)
  int64_t ldI, ldO;
  float* What;      // d_out x d_in
  uint8_t* codes;   // d_out x d_in
  int64_t d_out, d_in;
  const float* scale;
  const float* zero;
  float maxq;
  int s, I_lo;
  int ntile;        // workgroups [0, ntile) are this step's tiles
  // the far feedback of the previous step (tiles (I, ps - I), I in
  // [p_I_lo, p_I_lo + p_cnt)), spread over the workgroups from ntile on:
  // p_qr (p_qc) target blocks per tile at most for the row (column) kind
  int ps, p_I_lo, p_cnt, p_qr, p_qc, nfar;
  int mt, nt;       // tile counts of the padded matrices
};

// acc += op(A) B with K = YT for this wave's 32 x 32 block at (wm, wn), both
// operands in LDS: A(m, k) = Ap[m][k] if AT else Ap[k][m]; B(k, n) = Bp[k][n].
// acc[r] of lane (lr, lk) is element (wm + 8 (r / 4) + 4 lk + r % 4, wn + lr).
template <bool AT>
__device__ inline void mfma_k64(const float (*Ap)[YP], const float (*Bp)[YP], f32x16& acc, int wm,
                                int wn, int lr, int lk) {
#pragma unroll
  for (int kk = 0; kk < YT; kk += 2) {
    const float av = AT ? Ap[wm + lr][kk + lk] : Ap[kk + lk][wm + lr];
    const float bv = Bp[kk + lk][wn + lr];
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
  }
}

// The far feedback of the previous step's tiles, as 64 x 64 x 64 products on
// the CUs that this step's tiles leave free:
//   row kind:    M[I, c] += e_IJ U_I[J, c]        for column blocks c >= J + 2
//   column kind: Wk[r, J] -= U_O[I, r]^T M_IJ     for row blocks r >= I + 2
// Task q of tile b targets block J + 2 + q (row kind) or I + 2 + q (column
// kind); tasks past the matrix are skipped. Nothing here touches what this
// step's tiles read or write: their blocks lie on the anti-diagonal
// I + J = ps + 1, the targets at least one block beyond it. The next task's
// operands are loaded while the current one multiplies.
__device__ inline bool far_valid(const YaqaStep& a, int idx, int nrow) {
  if (idx < nrow) {
    const int b = idx / a.p_qr, q = idx % a.p_qr;
    const int J = a.ps - (a.p_I_lo + b);
    return J + 2 + q < a.nt;
  }
  const int b = (idx - nrow) / a.p_qc, q = (idx - nrow) % a.p_qc;
  return a.p_I_lo + b + 2 + q < a.mt;
}

struct FarOps {
  const float* A;  // row kind [m][k], column kind [k][m]
  const float* B;  // [k][n]
  float* C;        // output block, row stride ld
  int64_t lda, ldb;
};

__device__ inline FarOps far_ops(const YaqaStep& a, int idx, int nrow) {
  FarOps o;
  if (idx < nrow) {
    const int b = idx / a.p_qr, q = idx % a.p_qr;
    const int I = a.p_I_lo + b, J = a.ps - I, c = J + 2 + q;
    o.A = a.E + int64_t(I) * YT * a.ld + int64_t(J) * YT;
    o.lda = a.ld;
    o.B = a.UI + int64_t(J) * YT * a.ldI + int64_t(c) * YT;
    o.ldb = a.ldI;
    o.C = a.Mp + int64_t(I) * YT * a.ld + int64_t(c) * YT;
  } else {
    const int b = (idx - nrow) / a.p_qc, q = (idx - nrow) % a.p_qc;
    const int I = a.p_I_lo + b, J = a.ps - I, r = I + 2 + q;
    o.A = a.UO + int64_t(I) * YT * a.ldO + int64_t(r) * YT;
    o.lda = a.ldO;
    o.B = a.Mp + int64_t(I) * YT * a.ld + int64_t(J) * YT;
    o.ldb = a.ld;
    o.C = a.Wk + int64_t(r) * YT * a.ld + int64_t(J) * YT;
  }
  return o;
}

__device__ inline int far_next(const YaqaStep& a, int idx, int nrow, int ntot) {
  while (idx < ntot && !far_valid(a, idx, nrow)) idx += a.nfar;
  return idx;
}

constexpr int FNV = YT * YT / 4 / 256;  // float4 per thread and block

static_assert(FNV == 4, "far-task operand registers are written out for 4 float4 per block");

// 4 float4 of each operand block per thread, as named registers (arrays of
// them carried around the task loop were placed in scratch memory)
struct FarRegs {
  float4 a0, a1, a2, a3, b0, b1, b2, b3;
};

__device__ inline FarRegs far_load(const FarOps& o) {
  const int t = threadIdx.x;
  const int row = t / (YT / 4), col = 4 * (t % (YT / 4));  // element t; t + 256 h is 16 h rows down
  const float* pa = o.A + row * o.lda + col;
  const float* pb = o.B + row * o.ldb + col;
  FarRegs v;
  v.a0 = *reinterpret_cast<const float4*>(pa);
  v.a1 = *reinterpret_cast<const float4*>(pa + 16 * o.lda);
  v.a2 = *reinterpret_cast<const float4*>(pa + 32 * o.lda);
  v.a3 = *reinterpret_cast<const float4*>(pa + 48 * o.lda);
  v.b0 = *reinterpret_cast<const float4*>(pb);
  v.b1 = *reinterpret_cast<const float4*>(pb + 16 * o.ldb);
  v.b2 = *reinterpret_cast<const float4*>(pb + 32 * o.ldb);
  v.b3 = *reinterpret_cast<const float4*>(pb + 48 * o.ldb);
  return v;
}

__device__ __attribute__((always_inline)) inline void far_tasks(const YaqaStep& a, int f, float* sm) {
  float(*As)[YP] = reinterpret_cast<float(*)[YP]>(sm);
  float(*Bs)[YP] = reinterpret_cast<float(*)[YP]>(sm + YT * YP);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int lr = lane & 31, lk = lane >> 5;
  const int wm = (w >> 1) * 32, wn = (w & 1) * 32;
  const int nrow = a.p_cnt * a.p_qr;
  const int ntot = nrow + a.p_cnt * a.p_qc;
  int idx = far_next(a, f, nrow, ntot);
  if (idx >= ntot) return;
  FarRegs v = far_load(far_ops(a, idx, nrow));
  while (idx < ntot) {
    __syncthreads();  // the previous task's LDS reads are done
    {
      const int row = t / (YT / 4), col = 4 * (t % (YT / 4));
      *reinterpret_cast<float4*>(&As[row][col]) = v.a0;
      *reinterpret_cast<float4*>(&As[row + 16][col]) = v.a1;
      *reinterpret_cast<float4*>(&As[row + 32][col]) = v.a2;
      *reinterpret_cast<float4*>(&As[row + 48][col]) = v.a3;
      *reinterpret_cast<float4*>(&Bs[row][col]) = v.b0;
      *reinterpret_cast<float4*>(&Bs[row + 16][col]) = v.b1;
      *reinterpret_cast<float4*>(&Bs[row + 32][col]) = v.b2;
      *reinterpret_cast<float4*>(&Bs[row + 48][col]) = v.b3;
    }
    __syncthreads();
    const bool rowk = idx < nrow;
    float* C = far_ops(a, idx, nrow).C;
    float cv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) cv[r] = C[(wm + 8 * (r >> 2) + 4 * lk + (r & 3)) * a.ld + wn + lr];
    const int nidx = far_next(a, idx + a.nfar, nrow, ntot);
    // after the last task this reloads the current one (unused)
    v = far_load(far_ops(a, nidx < ntot ? nidx : idx, nrow));
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    if (rowk) mfma_k64<true>(As, Bs, acc, wm, wn, lr, lk);
    else mfma_k64<false>(As, Bs, acc, wm, wn, lr, lk);
    const float alpha = rowk ? 1.f : -1.f;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      C[(wm + 8 * (r >> 2) + 4 * lk + (r & 3)) * a.ld + wn + lr] = cv[r] + alpha * acc[r];
    idx = nidx;
  }
}

// One tile (I, J) of the wavefront. Besides the far feedback already in Wk
// and Mp it takes the near feedback of its two finished neighbours itself:
//   P2 = e_{I,J-1} U_I[J-1, J]           (completes Mpart_IJ)
//   P1 = U_O[I-1, I]^T M_{I-1, J}        (M of the tile above, complete)
//   Z0 = Wk_IJ - P1 - U_O[I, I]^T (Mpart_IJ + P2)
// as fp32 MFMA products over K = 64 in LDS, then sweeps the tile and writes
// e, W^, the codes and its complete M = Mpart + P2 + e_IJ U_I[J, J].
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void yaqa_tile_kernel(
    YaqaStep a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  if (int(blockIdx.x) >= a.ntile) {
    far_tasks(a, int(blockIdx.x) - a.ntile, sm);
    return;
  }
  float(*UIs)[YP] = reinterpret_cast<float(*)[YP]>(sm);               // U_I[l][c], 0 for c < l
  float(*UOt)[YP] = reinterpret_cast<float(*)[YP]>(sm + YT * YP);     // U_O[k][i] at [i][k], 0 for k > i
  float(*Ms)[YP] = reinterpret_cast<float(*)[YP]>(sm + 2 * YT * YP);  // Mpart (+ P2)
  float(*Es)[YP] = reinterpret_cast<float(*)[YP]>(sm + 3 * YT * YP);  // staged e
  float(*A1)[YP] = reinterpret_cast<float(*)[YP]>(sm + 4 * YT * YP);  // e_{I,J-1}, then staged T
  float(*B1)[YP] = reinterpret_cast<float(*)[YP]>(sm + 5 * YT * YP);  // U_I[J-1,J], then staged W^
  float(*A2)[YP] = reinterpret_cast<float(*)[YP]>(sm + 6 * YT * YP);  // U_O[I-1,I]
  float(*B2)[YP] = reinterpret_cast<float(*)[YP]>(sm + 7 * YT * YP);  // M_{I-1,J}, then Z
  float* uiinv = sm + 8 * YT * YP;                                    // 1 / U_I[j][j]
  float* erow = uiinv + YT;                                           // [2][YT]
  float* tcol = erow + 2 * YT;                                        // [2][YT]
  uint8_t(*Cs)[YCP] = reinterpret_cast<uint8_t(*)[YCP]>(tcol + 2 * YT);

  const int t = threadIdx.x;
  const int I = a.I_lo + int(blockIdx.x);
  const int J = a.s - I;
  const int64_t r0 = int64_t(I) * YT, c0 = int64_t(J) * YT;
  const int lane = t & 63, w = t >> 6;
  const int lr = lane & 31, lk = lane >> 5;
  const int wm = (w >> 1) * 32, wn = (w & 1) * 32;
  const int i = t / YNSEG;
  const int cb = (t % YNSEG) * YSEG;
  const int64_t grow = r0 + i;

  // every operand block in flight at once: the diagonal blocks of U_I and
  // U_O, Mpart, this thread's Wk, and the two neighbours' operands
  constexpr int NB = YT * YT / 4 / 256;  // float4 per thread and block
  float4 gUI[NB], gUO[NB], gM[NB], gEL[NB], gUIo[NB], gUOo[NB], gMa[NB], wk[YSEG / 4];
  const int64_t cl = J > 0 ? c0 - YT : c0, ru = I > 0 ? r0 - YT : r0;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int e4 = t + 256 * k;
    const int r = e4 / (YT / 4), c = (e4 % (YT / 4)) * 4;
    gUI[k] = *reinterpret_cast<const float4*>(a.UI + (c0 + r) * a.ldI + c0 + c);
    gUO[k] = *reinterpret_cast<const float4*>(a.UO + (r0 + r) * a.ldO + r0 + c);
    gM[k] = *reinterpret_cast<const float4*>(a.Mp + (r0 + r) * a.ld + c0 + c);
    // without a left or upper neighbour these read the tile's own blocks
    // (in bounds, unused)
    gEL[k] = *reinterpret_cast<const float4*>(a.E + (r0 + r) * a.ld + cl + c);
    gUIo[k] = *reinterpret_cast<const float4*>(a.UI + (cl + r) * a.ldI + c0 + c);
    gUOo[k] = *reinterpret_cast<const float4*>(a.UO + (ru + r) * a.ldO + r0 + c);
    gMa[k] = *reinterpret_cast<const float4*>(a.Mp + (ru + r) * a.ld + c0 + c);
  }
#pragma unroll
  for (int j = 0; j < YSEG / 4; ++j)
    wk[j] = *reinterpret_cast<const float4*>(a.Wk + grow * a.ld + c0 + cb + 4 * j);
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int e4 = t + 256 * k;
    const int r = e4 / (YT / 4), c = (e4 % (YT / 4)) * 4;
    float4 ui = gUI[k];
    ui.x = c >= r ? ui.x : 0.f;
    ui.y = c + 1 >= r ? ui.y : 0.f;
    ui.z = c + 2 >= r ? ui.z : 0.f;
    ui.w = c + 3 >= r ? ui.w : 0.f;
    *reinterpret_cast<float4*>(&UIs[r][c]) = ui;
    const float4 uo = gUO[k];
    UOt[c][r] = c >= r ? uo.x : 0.f;
    UOt[c + 1][r] = c + 1 >= r ? uo.y : 0.f;
    UOt[c + 2][r] = c + 2 >= r ? uo.z : 0.f;
    UOt[c + 3][r] = c + 3 >= r ? uo.w : 0.f;
    *reinterpret_cast<float4*>(&Ms[r][c]) = gM[k];
    *reinterpret_cast<float4*>(&A1[r][c]) = gEL[k];   // e_{I,J-1} as [m][k]
    *reinterpret_cast<float4*>(&B1[r][c]) = gUIo[k];  // U_I[J-1, J] as [k][n]
    *reinterpret_cast<float4*>(&A2[r][c]) = gUOo[k];  // U_O[I-1, I] as [k][m]
    *reinterpret_cast<float4*>(&B2[r][c]) = gMa[k];   // M_{I-1, J}
  }
  if (t < 4 * YT) erow[t] = 0.f;  // erow and tcol (contiguous)
  __syncthreads();
  if (t < YT) uiinv[t] = 1.f / UIs[t][t];

  // P2 into Mpart; P1 + U_O[I,I]^T (Mpart + P2) into acc
  f32x16 acc, acc2;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    acc[r] = 0.f;
    acc2[r] = 0.f;
  }
  if (J > 0) mfma_k64<true>(A1, B1, acc2, wm, wn, lr, lk);
  if (I > 0) mfma_k64<false>(A2, B2, acc, wm, wn, lr, lk);
  if (J > 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) Ms[wm + 8 * (r >> 2) + 4 * lk + (r & 3)][wn + lr] += acc2[r];
  }
  __syncthreads();
  mfma_k64<true>(UOt, Ms, acc, wm, wn, lr, lk);
#pragma unroll
  for (int r = 0; r < 16; ++r) B2[wm + 8 * (r >> 2) + 4 * lk + (r & 3)][wn + lr] = acc[r];
  __syncthreads();

  float sc = 1.f, zr = 0.f;  // padded rows: any finite grid
  if (grow < a.d_out) {
    sc = a.scale[grow];
    zr = a.zero[grow];
  }
  const float isc = 1.f / sc;
  const float uo = UOt[i][i];
  const float iuo = 1.f / uo;

  float v[YSEG], tt[YSEG], tcp[YSEG], uic[YSEG], win[8];
  {
#pragma unroll
    for (int j = 0; j < YSEG; j += 4) {
      const float4 x = wk[j / 4];
      const float4 z = *reinterpret_cast<const float4*>(&B2[i][cb + j]);
      v[j] = x.x - z.x;
      v[j + 1] = x.y - z.y;
      v[j + 2] = x.z - z.z;
      v[j + 3] = x.w - z.w;
    }
#pragma unroll
    for (int j = 0; j < YSEG; ++j) {
      tt[j] = 0.f;
      tcp[j] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) win[k] = 0.f;
  }
  // U_I row and 1 / U_I[j][j] of this row's front at the first step
  float uinv;
  {
    const int j0 = -2 * i;
    const int jc = j0 >= 0 && j0 < YT ? j0 : 0;
#pragma unroll
    for (int j = 0; j < YSEG; j += 4) {
      const float4 u = *reinterpret_cast<const float4*>(&UIs[jc][cb + j]);
      uic[j] = u.x;
      uic[j + 1] = u.y;
      uic[j + 2] = u.z;
      uic[j + 3] = u.w;
    }
    uinv = uiinv[jc];
  }
  __syncthreads();  // A1 and B1 are free for the staged T and W^

  // Row i reaches column j at step 2 i + j. Along a row the chain stays in
  // registers (the front's e reaches the row's four lanes by DPP quad sums);
  // the column feedback T of step sp is read from LDS after the step's
  // barrier and applied during step sp + 1, one step before the row below
  // reaches that column. The window win[k % 8] = U_O[k][i] holds the
  // coefficients of the last eight producer rows; with the step loop
  // unrolled by 16 (and sp0 a multiple of 16) every slot index below is a
  // compile-time constant.
  constexpr int NSTEP = 2 * (YT - 1) + YT;
#pragma unroll 1
  for (int sp0 = 0; sp0 < NSTEP; sp0 += 16) {
#pragma unroll
    for (int p = 0; p < 16; ++p) {
      const int sp = sp0 + p;
      float* tb = tcol + (p & 1) * YT;
      const int j0 = sp - 2 * i;
      const int jj = j0 - cb;
      float ev = 0.f;
      if (jj >= 0 && jj < YSEG) {
        // the front entry of this row: a 4-level tree of bitwise selects
        // (written as masks: a select tree on the index is turned back into
        // an indexed private array, which would live in scratch memory)
        auto pick = [](float lo, float hi, int m) {
          return __int_as_float((__float_as_int(lo) & ~m) | (__float_as_int(hi) & m));
        };
        const int m0 = -(jj & 1), m1 = -((jj >> 1) & 1), m2 = -((jj >> 2) & 1), m3 = -((jj >> 3) & 1);
        float x8[8], t8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          x8[k] = pick(v[2 * k], v[2 * k + 1], m0);
          t8[k] = pick(tt[2 * k], tt[2 * k + 1], m0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          x8[k] = pick(x8[2 * k], x8[2 * k + 1], m1);
          t8[k] = pick(t8[2 * k], t8[2 * k + 1], m1);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          x8[k] = pick(x8[2 * k], x8[2 * k + 1], m2);
          t8[k] = pick(t8[2 * k], t8[2 * k + 1], m2);
        }
        const float vz = pick(x8[0], x8[1], m3);
        const float ta = pick(t8[0], t8[1], m3);
        const float z = vz - uo * ta;
        const float q = __builtin_amdgcn_fmed3f(rintf(z * isc) + zr, 0.f, a.maxq);
        const float wq = sc * (q - zr);
        const float eps = z - wq;
        ev = eps * iuo * uinv;
        const float tv = ta + eps * iuo;
        tb[j0] = tv;
        A1[i][j0] = tv;
        B1[i][j0] = wq;
        Es[i][j0] = ev;
        Cs[i][j0] = uint8_t(q);
      }
      // e of the row's front to its four lanes (the others hold 0)
      ev += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ev), 0xB1, 0xF, 0xF, true));
      ev += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ev), 0x4E, 0xF, 0xF, true));
#pragma unroll
      for (int j = 0; j < YSEG; ++j) tt[j] += ev * uic[j];
      // column feedback produced at step sp - 1: column cb + j from row
      // (sp - 1 - cb - j) / 2, present only for one parity of j
#pragma unroll
      for (int j = 0; j < YSEG; ++j)
        if (((p - 1 - j) & 1) == 0) v[j] -= win[((p - 1 - j) >> 1) & 7] * tcp[j];
      __syncthreads();
      // for step sp + 1: this step's T, the newest window entry, the next
      // U_I row and 1 / U_I[j][j] of the front
#pragma unroll
      for (int j = 0; j < YSEG; j += 4) {
        const float4 tc = *reinterpret_cast<const float4*>(tb + cb + j);
        tcp[j] = tc.x;
        tcp[j + 1] = tc.y;
        tcp[j + 2] = tc.z;
        tcp[j + 3] = tc.w;
      }
      {
        const int k = (sp - cb) >> 1;  // newest producer row of a column of this lane
        const bool in = k >= 0 && k < YT;
        const float x = UOt[i][in ? k : 0];
        win[(p >> 1) & 7] = in ? x : 0.f;
      }
      {
        const int jn = j0 + 1;
        const int jc = jn >= 0 && jn < YT ? jn : 0;
#pragma unroll
        for (int j = 0; j < YSEG; j += 4) {
          const float4 u = *reinterpret_cast<const float4*>(&UIs[jc][cb + j]);
          uic[j] = u.x;
          uic[j + 1] = u.y;
          uic[j + 2] = u.z;
          uic[j + 3] = u.w;
        }
        uinv = uiinv[jc];
      }
    }
  }
  __syncthreads();

  // results: e and the complete M into the padded buffers, W^ and codes into
  // the real outputs
  for (int e4 = t; e4 < YT * YT / 4; e4 += 256) {
    const int r = e4 / (YT / 4), c = (e4 % (YT / 4)) * 4;
    *reinterpret_cast<float4*>(a.E + (r0 + r) * a.ld + c0 + c) =
        *reinterpret_cast<const float4*>(&Es[r][c]);
    const float4 m = *reinterpret_cast<const float4*>(&Ms[r][c]);
    const float4 tv = *reinterpret_cast<const float4*>(&A1[r][c]);
    *reinterpret_cast<float4*>(a.Mp + (r0 + r) * a.ld + c0 + c) =
        make_float4(m.x + tv.x, m.y + tv.y, m.z + tv.z, m.w + tv.w);
  }
  for (int e = t; e < YT * YT; e += 256) {
    const int r = e / YT, c = e % YT;
    const int64_t gr = r0 + r, gc = c0 + c;
    if (gr < a.d_out && gc < a.d_in) {
      a.What[gr * a.d_in + gc] = B1[r][c];
      a.codes[gr * a.d_in + gc] = Cs[r][c];
    }
  }
}

// dst (rows_p x cols_p, row stride cols_p) = src (rows x cols, row stride
// lds) padded with zeros, or with ones on the padded diagonal
__global__ __launch_bounds__(256) void pad_copy_kernel(const float* __restrict__ src, int64_t rows,
                                                       int64_t cols, int64_t lds, float* dst,
                                                       int64_t rows_p, int64_t cols_p, int diag_one) {
  for (int64_t r = blockIdx.y; r < rows_p; r += gridDim.y)
    for (int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x; c < cols_p;
         c += int64_t(gridDim.x) * 256) {
      float v;
      if (r < rows && c < cols) v = src[r * lds + c];
      else v = (diag_one && r == c) ? 1.f : 0.f;
      dst[r * cols_p + c] = v;
    }
}

kq_status pad_copy(const float* src, int64_t rows, int64_t cols, float* dst, int64_t rows_p,
                   int64_t cols_p, bool diag_one, hipStream_t s) {
  dim3 grid(unsigned(std::min<int64_t>(cdiv(cols_p, 256), 32)),
            unsigned(std::min<int64_t>(rows_p, 65535)));
  pad_copy_kernel<<<grid, 256, 0, s>>>(src, rows, cols, cols, dst, rows_p, cols_p, diag_one ? 1 : 0);
  KQ_HIP(hipGetLastError());
  return KQ_OK;
}

inline int64_t pad_to(int64_t x) { return cdiv(x, YT) * YT; }

}  // namespace

size_t yaqa_ws_bytes(int64_t d_out, int64_t d_in, bool has_d) {
  const int64_t mp = pad_to(d_out), np = pad_to(d_in);
  Arena ar{nullptr, 0, 0};
  ar.take<float>(size_t(mp) * np);  // Wk
  ar.take<float>(size_t(mp) * np);  // M
  ar.take<float>(size_t(mp) * np);  // E
  if (np != d_in) ar.take<float>(size_t(np) * np);  // padded U_in
  if (mp != d_out) ar.take<float>(size_t(mp) * mp);  // padded U_out
  if (has_d) {
    if (np != d_in) ar.take<float>(size_t(np) * np);  // padded D
    ar.take<float>(size_t(np) * np);                  // P
    ar.take<float>(size_t(np) * np);                  // T inside form_p
  }
  return ar.used;
}

kq_status yaqa_run(float* W, const float* U_in, const float* U_out, const float* D, int64_t d_out,
                   int64_t d_in, int bits, uint8_t* codes, float* scale, float* zero, Arena& ws,
                   hipStream_t s) {
  const int64_t mp = pad_to(d_out), np = pad_to(d_in);
  const int mt = int(mp / YT), nt = int(np / YT);
  float* Wk = ws.take<float>(size_t(mp) * np);
  float* Mp = ws.take<float>(size_t(mp) * np);
  float* E = ws.take<float>(size_t(mp) * np);
  if (!Wk || !Mp || !E) return fail(KQ_ERR_WORKSPACE, "yaqa_quantize: workspace too small");
  const float* UI = U_in;
  const float* UO = U_out;
  if (np != d_in) {
    float* p = ws.take<float>(size_t(np) * np);
    if (!p) return fail(KQ_ERR_WORKSPACE, "yaqa_quantize: workspace too small");
    KQ_TRY(pad_copy(U_in, d_in, d_in, p, np, np, true, s));
    UI = p;
  }
  if (mp != d_out) {
    float* p = ws.take<float>(size_t(mp) * mp);
    if (!p) return fail(KQ_ERR_WORKSPACE, "yaqa_quantize: workspace too small");
    KQ_TRY(pad_copy(U_out, d_out, d_out, p, mp, mp, true, s));
    UO = p;
  }
  KQ_TRY(pad_copy(W, d_out, d_in, Wk, mp, np, false, s));
  // one grid per output channel from W0 (the zero padding leaves min(., 0)
  // and max(., 0) unchanged)
  KQ_TRY(grid_rows(Wk, d_out, np, float((1 << bits) - 1), scale, zero, s));
  if (D) {
    const float* Dp = D;
    if (np != d_in) {
      float* p = ws.take<float>(size_t(np) * np);
      if (!p) return fail(KQ_ERR_WORKSPACE, "yaqa_quantize: workspace too small");
      KQ_TRY(pad_copy(D, d_in, d_in, p, np, np, false, s));
      Dp = p;
    }
    float* P = ws.take<float>(size_t(np) * np);
    if (!P) return fail(KQ_ERR_WORKSPACE, "yaqa_quantize: workspace too small");
    KQ_TRY(formp_run(Dp, UI, np, P, ws, s));
    // target W* = W0 + W0 P into M's buffer, then swap the two
    GemmArgs gf = gemm_args(Wk, np, P, np, Mp, np, mp, np, np, 1.f, 1.f, G_B_UPPER | G_ORDER_NDESC);
    gf.Cin = Wk;
    KQ_TRY(gemm_f32(gf, s));
    std::swap(Wk, Mp);
  }
  KQ_TRY(fill_f32(Mp, mp * np, 0.f, s));

  YaqaStep st{};
  st.Wk = Wk;
  st.Mp = Mp;
  st.E = E;
  st.ld = np;
  st.UI = UI;
  st.UO = UO;
  st.ldI = np;
  st.ldO = mp;
  st.What = W;
  st.codes = codes;
  st.d_out = d_out;
  st.d_in = d_in;
  st.scale = scale;
  st.zero = zero;
  st.maxq = float((1 << bits) - 1);
  KQ_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(yaqa_tile_kernel),
                             hipFuncAttributeMaxDynamicSharedMemorySize, int(YAQA_LDS)));

  // One launch per step, on the caller's stream: the tiles of step s, and on
  // the CUs they leave free the far feedback of step s - 1, which the tiles
  // of step s + 1 are the first to need.
  int ncu = 0;
  {
    int dev = 0;
    KQ_HIP(hipGetDevice(&dev));
    KQ_HIP(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  }
  st.mt = mt;
  st.nt = nt;
  const int nsteps = mt + nt - 1;
  for (int sidx = 0; sidx < nsteps; ++sidx) {
    const int I_lo = std::max(0, sidx - nt + 1), I_hi = std::min(sidx, mt - 1);
    const int cnt = I_hi - I_lo + 1;
    st.s = sidx;
    st.I_lo = I_lo;
    st.ntile = cnt;
    st.nfar = 0;
    st.p_cnt = 0;
    if (sidx > 0) {
      const int ps = sidx - 1;
      const int pI_lo = std::max(0, ps - nt + 1), pI_hi = std::min(ps, mt - 1);
      st.ps = ps;
      st.p_I_lo = pI_lo;
      st.p_cnt = pI_hi - pI_lo + 1;
      // the tile with the smallest J (the largest I) has the most row-kind
      // targets, the one with the smallest I the most column-kind targets
      st.p_qr = std::max(0, nt - 2 - (ps - pI_hi));
      st.p_qc = std::max(0, mt - 2 - pI_lo);
      const int64_t space = int64_t(st.p_cnt) * (st.p_qr + st.p_qc);
      if (space > 0) st.nfar = int(std::min<int64_t>(space, std::max(64, ncu - cnt)));
    }
    yaqa_tile_kernel<<<unsigned(cnt + st.nfar), 256, YAQA_LDS, s>>>(st);
    KQ_HIP(hipGetLastError());
  }
  return KQ_OK;
}

}  // namespace kq
