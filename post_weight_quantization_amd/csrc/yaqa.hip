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
// Order used here: a wavefront over TS x TS tiles. The tiles (I, J) with
// I + J = s form one launch, one workgroup per tile, and inside a tile the
// entries run as a skewed wavefront (row i reaches column j at step i + j).
// What a tile needs from outside arrives through two accumulators in HBM:
//   M[I,J] = sum_{L<=J} e_{I,L} U_I[L,J]            (row feedback)
//   Wk     = W* - sum_{K<I} U_O[K,I]^T M[K,J]          (column feedback)
// so a tile starts from Z0 = Wk_IJ - U_O[I,I]^T Mpart_IJ, Mpart holding the
// column blocks L < J. After each step two batched fp32 MFMA GEMMs carry its
// results on: M[I, :] += e_IJ U_I[J, :] (U_I upper: only blocks >= J change,
// and block J becomes the complete M_IJ), then
// Wk[:, J] -= U_O[I, :]^T M_IJ (only row blocks >= I change).
//
// Inside a tile, thread (row i, 16-column segment) keeps v = Z0 - (column
// feedback received) and t = sum_{l<j} e_il U_I[l,j] for its 16 columns, so
// z = v - U_O[i,i] t. At each step the entry on the front of each row is
// rounded; its e goes to its row (t += e U_I[j, :]) and its
// T = t + (z - w^) / U_O[i,i] (= sum_{l<=j} e_il U_I[l,j]) down its column
// (v -= U_O[i, r] T for rows r below). Both travel through LDS, double
// buffered by step parity, with one barrier per step. The column
// coefficients U_O[sp - c][i] of a thread's 16 columns form a sliding window
// that takes one LDS read per step: with the step loop unrolled by 16 the
// window slot of each column is a compile-time index.
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

constexpr size_t YAQA_LDS = sizeof(float) * (4 * YT * YP + YT + 4 * YT) + YT * YCP;

struct YaqaStep {
  const float* Wk;  // m_p x n_p working input (column feedback applied)
  const float* Mp;  // m_p x n_p row-feedback accumulator
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
};

__global__ __launch_bounds__(256) void yaqa_tile_kernel(YaqaStep a) {
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float(*UIs)[YP] = reinterpret_cast<float(*)[YP]>(sm);               // U_I[l][c], 0 for c < l
  float(*UOt)[YP] = reinterpret_cast<float(*)[YP]>(sm + YT * YP);     // U_O[k][i] at [i][k], 0 for k > i
  float(*Ms)[YP] = reinterpret_cast<float(*)[YP]>(sm + 2 * YT * YP);  // Mpart, then staged W^
  float(*Es)[YP] = reinterpret_cast<float(*)[YP]>(sm + 3 * YT * YP);  // staged e
  float* uiinv = sm + 4 * YT * YP;                                    // 1 / U_I[j][j]
  float* erow = uiinv + YT;                                           // [2][YT]
  float* tcol = erow + 2 * YT;                                        // [2][YT]
  uint8_t(*Cs)[YCP] = reinterpret_cast<uint8_t(*)[YCP]>(tcol + 2 * YT);

  const int t = threadIdx.x;
  const int I = a.I_lo + int(blockIdx.x);
  const int J = a.s - I;
  const int64_t r0 = int64_t(I) * YT, c0 = int64_t(J) * YT;

  for (int e4 = t; e4 < YT * YT / 4; e4 += 256) {
    const int r = e4 / (YT / 4), c = (e4 % (YT / 4)) * 4;
    float4 ui = *reinterpret_cast<const float4*>(a.UI + (c0 + r) * a.ldI + c0 + c);
    ui.x = c >= r ? ui.x : 0.f;
    ui.y = c + 1 >= r ? ui.y : 0.f;
    ui.z = c + 2 >= r ? ui.z : 0.f;
    ui.w = c + 3 >= r ? ui.w : 0.f;
    *reinterpret_cast<float4*>(&UIs[r][c]) = ui;
    const float4 uo = *reinterpret_cast<const float4*>(a.UO + (r0 + r) * a.ldO + r0 + c);
    UOt[c][r] = c >= r ? uo.x : 0.f;
    UOt[c + 1][r] = c + 1 >= r ? uo.y : 0.f;
    UOt[c + 2][r] = c + 2 >= r ? uo.z : 0.f;
    UOt[c + 3][r] = c + 3 >= r ? uo.w : 0.f;
    *reinterpret_cast<float4*>(&Ms[r][c]) =
        *reinterpret_cast<const float4*>(a.Mp + (r0 + r) * a.ld + c0 + c);
  }
  if (t < 4 * YT) erow[t] = 0.f;  // erow and tcol (contiguous)
  __syncthreads();
  if (t < YT) uiinv[t] = 1.f / UIs[t][t];

  const int i = t / YNSEG;
  const int cb = (t % YNSEG) * YSEG;
  const int64_t grow = r0 + i;
  float sc = 1.f, zr = 0.f;  // padded rows: any finite grid
  if (grow < a.d_out) {
    sc = a.scale[grow];
    zr = a.zero[grow];
  }
  const float isc = 1.f / sc;
  const float uo = UOt[i][i];
  const float iuo = 1.f / uo;

  // Z0 = Wk_IJ - U_O[I,I]^T Mpart_IJ for this thread's columns; U_O[k][i] = 0
  // for k > i, so the wave stops at its last row
  float v[YSEG], tt[YSEG], win[YSEG];
  {
    const float* wp = a.Wk + grow * a.ld + c0 + cb;
#pragma unroll
    for (int j = 0; j < YSEG; j += 4) {
      const float4 x = *reinterpret_cast<const float4*>(wp + j);
      v[j] = x.x;
      v[j + 1] = x.y;
      v[j + 2] = x.z;
      v[j + 3] = x.w;
    }
    const int kend = (t / 64 + 1) * (64 / YNSEG);
    for (int k = 0; k < kend; ++k) {
      const float co = UOt[i][k];
#pragma unroll
      for (int j = 0; j < YSEG; j += 4) {
        const float4 m = *reinterpret_cast<const float4*>(&Ms[k][cb + j]);
        v[j] -= co * m.x;
        v[j + 1] -= co * m.y;
        v[j + 2] -= co * m.z;
        v[j + 3] -= co * m.w;
      }
    }
#pragma unroll
    for (int j = 0; j < YSEG; ++j) {
      tt[j] = 0.f;
      win[j] = 0.f;
    }
  }
  __syncthreads();  // Ms is free for the staged W^

  constexpr int NSTEP = 2 * YT - 1;
#pragma unroll 1
  for (int sp0 = 0; sp0 < NSTEP; sp0 += YSEG) {
#pragma unroll
    for (int p = 0; p < YSEG; ++p) {
      const int sp = sp0 + p;
      float* eb = erow + (p & 1) * YT;
      float* tb = tcol + (p & 1) * YT;
      const int j0 = sp - i;
      const int jj = j0 - cb;
      if (jj >= 0 && jj < YSEG) {
        float vz = v[0], ta = tt[0];
#pragma unroll
        for (int k = 1; k < YSEG; ++k) {
          vz = jj == k ? v[k] : vz;
          ta = jj == k ? tt[k] : ta;
        }
        const float z = vz - uo * ta;
        const float q = __builtin_amdgcn_fmed3f(rintf(z * isc) + zr, 0.f, a.maxq);
        const float wq = sc * (q - zr);
        const float eps = z - wq;
        const float e = eps * iuo * uiinv[j0];
        eb[i] = e;
        tb[j0] = ta + eps * iuo;
        Ms[i][j0] = wq;
        Es[i][j0] = e;
        Cs[i][j0] = uint8_t(q);
      }
      __syncthreads();
      {
        const int k = sp - cb;  // newest window entry U_O[k][i]
        const bool in = k >= 0 && k < YT;
        const float x = UOt[i][in ? k : 0];
        win[p] = in ? x : 0.f;
      }
      const bool act = j0 >= 0 && j0 < YT;
      const float e = act ? eb[i] : 0.f;
      const int jr = act ? j0 : 0;
#pragma unroll
      for (int j = 0; j < YSEG; j += 4) {
        const float4 u = *reinterpret_cast<const float4*>(&UIs[jr][cb + j]);
        tt[j] += e * u.x;
        tt[j + 1] += e * u.y;
        tt[j + 2] += e * u.z;
        tt[j + 3] += e * u.w;
        const float4 tc = *reinterpret_cast<const float4*>(tb + cb + j);
        v[j] -= win[(p - j) & (YSEG - 1)] * tc.x;
        v[j + 1] -= win[(p - j - 1) & (YSEG - 1)] * tc.y;
        v[j + 2] -= win[(p - j - 2) & (YSEG - 1)] * tc.z;
        v[j + 3] -= win[(p - j - 3) & (YSEG - 1)] * tc.w;
      }
    }
  }
  __syncthreads();

  // results: e into the padded E, W^ and codes into the real outputs
  for (int e4 = t; e4 < YT * YT / 4; e4 += 256) {
    const int r = e4 / (YT / 4), c = (e4 % (YT / 4)) * 4;
    *reinterpret_cast<float4*>(a.E + (r0 + r) * a.ld + c0 + c) =
        *reinterpret_cast<const float4*>(&Es[r][c]);
  }
  for (int e = t; e < YT * YT; e += 256) {
    const int r = e / YT, c = e % YT;
    const int64_t gr = r0 + r, gc = c0 + c;
    if (gr < a.d_out && gc < a.d_in) {
      a.What[gr * a.d_in + gc] = Ms[r][c];
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
  for (int sidx = 0; sidx <= mt + nt - 2; ++sidx) {
    const int I_lo = std::max(0, sidx - nt + 1), I_hi = std::min(sidx, mt - 1);
    const int cnt = I_hi - I_lo + 1;
    const int J_hi = sidx - I_lo;
    st.s = sidx;
    st.I_lo = I_lo;
    yaqa_tile_kernel<<<unsigned(cnt), 256, YAQA_LDS, s>>>(st);
    KQ_HIP(hipGetLastError());
    // M[I, :] += e_IJ U_I[J, :]   (op(B) zero for global k > n: U_I upper)
    GemmArgs gr = gemm_args(E + int64_t(I_lo) * YT * np + int64_t(J_hi) * YT, np,
                            UI + int64_t(J_hi) * YT * np, np, Mp + int64_t(I_lo) * YT * np, np, YT,
                            np, YT, 1.f, 1.f, G_B_UPPER);
    gr.batch = cnt;
    gr.strideA = int64_t(YT) * np - YT;
    gr.strideB = -int64_t(YT) * np;
    gr.strideC = int64_t(YT) * np;
    gr.kbase = int64_t(J_hi) * YT;
    gr.kofs = -YT;
    KQ_TRY(gemm_f32(gr, s));
    // Wk[:, J] -= U_O[I, :]^T M_IJ   (op(A)[m][k] = U_O[I*YT + k][m], zero for global k > m)
    GemmArgs gc = gemm_args(UO + int64_t(I_lo) * YT * mp, mp,
                            Mp + int64_t(I_lo) * YT * np + int64_t(J_hi) * YT, np,
                            Wk + int64_t(J_hi) * YT, np, mp, YT, YT, -1.f, 1.f,
                            G_TRANS_A | G_A_LOWER);
    gc.batch = cnt;
    gc.strideA = int64_t(YT) * mp;
    gc.strideB = int64_t(YT) * np - YT;
    gc.strideC = -int64_t(YT);
    gc.kbase = int64_t(I_lo) * YT;
    gc.kofs = YT;
    KQ_TRY(gemm_f32(gc, s));
  }
  return KQ_OK;
}

}  // namespace kq
